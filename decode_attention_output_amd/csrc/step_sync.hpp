// Hand-over between the attention and the projection workgroups of one
// single-launch decode step.
//
// The attention side counts every finished sequence in its kv head's ready
// counter; each counter is kept kStepReplicas times, one per 128-byte line,
// so that each copy has only a few pollers. A projection workgroup waits until
// the copies it polls reach the number of sequences per kv head. The wait is
// bounded: a workgroup that gives up sets the error word (read back by
// decode_attn_step_status) and is told so, to poison its output. Every waiting
// workgroup then counts itself past its wait in two levels (32 counters, then
// one), so that no address takes more than a few dozen atomics; the last one
// checks that every copy of every ready counter is complete -- a copy that no
// workgroup polled may still have an increment in flight -- and only then
// returns them to zero for the next call.
#pragma once

#include "gfx950.hpp"
#include "kernels.hpp"

namespace da {

constexpr int kPassGroups = 32;

__device__ __forceinline__ uint32_t ready_load(const uint32_t* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 of a waiting workgroup: wait for kv heads [h0, h1] through copy
// `copy`. Returns false if the wait gave up (the error word is then set and
// acknowledged).
__device__ __forceinline__ bool ready_wait(const ReadySync& s, int h0, int h1, int copy) {
  uint32_t polls = 0;
  bool ok = true;
  for (int h = h0; h <= h1 && ok; ++h) {
    const uint32_t* c = &s.ready[(h * kStepReplicas + copy) * kCounterStride];
    while (ready_load(c) < s.target) {
      if (++polls >= s.wait_polls) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  if (!ok) {
    __hip_atomic_store(s.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_stores_done();  // the error word is in place before this workgroup counts itself past the wait
  }
  return ok;
}

// Thread 0 of waiting workgroup `w` (0 <= w < waiters), after ready_wait:
// count itself in its group. The returned count is only looked at later
// (ready_pass_last), so the atomic's round trip overlaps the workgroup's work.
__device__ __forceinline__ uint32_t ready_pass_sub(const ReadySync& s, int w) {
  return __hip_atomic_fetch_add(&s.pass_sub[w % kPassGroups], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0, with ready_pass_sub's result: true in the last workgroup past its wait.
__device__ __forceinline__ bool ready_pass_last(const ReadySync& s, int w, uint32_t prev_sub) {
  const int g = w % kPassGroups;
  const uint32_t in_group = (uint32_t)(s.waiters / kPassGroups + (g < s.waiters % kPassGroups ? 1 : 0));
  if (prev_sub != in_group - 1) return false;
  __hip_atomic_store(&s.pass_sub[g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t ngroups = (uint32_t)min(s.waiters, kPassGroups);
  if (__hip_atomic_fetch_add(s.pass_top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != ngroups - 1) return false;
  __hip_atomic_store(s.pass_top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Both steps at once: bit 0 if the wait gave up, bit 1 if this workgroup is
// the last one past its wait.
__device__ __forceinline__ uint32_t ready_wait_and_pass(const ReadySync& s, int h0, int h1, int copy, int w) {
  const bool ok = ready_wait(s, h0, h1, copy);
  const uint32_t prev = ready_pass_sub(s, w);
  return (ok ? 0u : 1u) | (ready_pass_last(s, w, prev) ? 2u : 0u);
}

// The whole workgroup, after a barrier that published ready_wait_and_pass's
// result: the last workgroup past its wait returns the ready counters to zero
// once every copy is complete, or leaves them and sets the error word.
__device__ __forceinline__ void ready_clear(const ReadySync& s, bool clearer) {
  if (!clearer) return;
  const int n = s.heads * kStepReplicas;
  bool done = ready_load(s.error) == 0u;
  for (int i = threadIdx.x; i < n && done; i += blockDim.x) {
    const uint32_t* c = &s.ready[i * kCounterStride];
    uint32_t polls = 0;
    while (ready_load(c) < s.target) {
      if (++polls >= s.wait_polls) {
        done = false;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  done = __syncthreads_and(done);
  if (done) {
    for (int i = threadIdx.x; i < n; i += blockDim.x)
      __hip_atomic_store(&s.ready[i * kCounterStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (threadIdx.x == 0) {
    __hip_atomic_store(s.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace da
