// Device helpers shared by the role-specialised decode kernels: explicit
// vector-memory waits, a barrier that leaves direct loads alone, direct
// global-to-LDS loads and the XCD-aware workgroup order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <utility>

#pragma clang diagnostic ignored "-Winline-asm"  // m0 is clobbered on purpose: the direct loads set it

namespace spmla {
namespace ws {

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left at
// their maxima).  The empty asm statements keep memory operations from being
// moved across the wait.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// Workgroup barrier: this wave's LDS reads and writes complete, then
// s_barrier.  No fence: direct loads in flight are left alone.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct loads into LDS: each lane's 16 (or 4) bytes at gptr land at LDS
// byte address lds + 16 * lane (4 * lane) of the issuing wave; lds must be
// the same in every lane.  Written as asm so that the compiler does not
// treat later LDS reads as waiting on them (it would wait for every load in
// flight); the waits are the explicit vm_wait calls.  An asm load issued
// before one of the compiler's own loads only makes the compiler's count
// for that load conservative, since loads complete in order.
// (An SALU write of M0 needs one wait state before an instruction that
// reads it for an LDS address; the compiler inserts no hazard padding inside
// asm, hence the s_nop.)  No memory clobber: the buffer a load fills is never
// the one being read in the same phase, and the waits and barriers around
// the loads carry the clobbers that order them.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds) : "m0");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds) : "m0");
}
template <class T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) T*)p);
}

// Logical workgroup index: the hardware deals workgroup ids round-robin over
// the 8 XCDs, so logical indices [x * n / 8, (x + 1) * n / 8) are given the
// ids that land on XCD x, and neighbours in the logical order share an L2.
__host__ __device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = bid & 7, slot = bid >> 3;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// Workgroup -> (request b, split s, head group hg) over a grid of
// batch * num_splits * n_hg workgroups.  Equal split counts: b-major over
// xcd_remap's logical order (a request's workgroups share an L2).  A fixed
// split length (spread): the (request, split) pairs go in split-major order,
// so that a ragged batch's empty tail splits are dispatched last, with the
// requests of split s rotated by s (pair p is split s = p / batch of request
// (p - s) mod batch), and are dealt to the XCDs round-robin, so that a
// request's splits land on consecutive XCDs and every XCD gets about an equal
// share of the pairs with work; the n_hg workgroups of a pair (they read the
// same rows) share an XCD: in each full round of 8 * n_hg ids, id i takes
// pair round * 8 + i % 8 and head group (i % (8 * n_hg)) / 8; the last,
// partial round takes its pairs in order.
struct WgCoord {
  int b, s, hg;
};
__host__ __device__ __forceinline__ WgCoord wg_coord(int bid, int n, int num_splits, int n_hg, bool spread) {
  if (!spread) {
    const int logical = xcd_remap(bid, n);
    return {logical / (n_hg * num_splits), (logical / n_hg) % num_splits, logical % n_hg};
  }
  const int batch = n / (num_splits * n_hg);
  const int full = batch * num_splits / 8;  // full rounds
  const int round_ids = 8 * n_hg;
  const int r = bid / round_ids, w = bid % round_ids;
  const int p = r < full ? r * 8 + (w & 7) : full * 8 + w / n_hg;
  const int hg = r < full ? w >> 3 : w % n_hg;
  const int s = p / batch;
  return {(p - s % batch + batch) % batch, s, hg};
}

}  // namespace ws
}  // namespace spmla
