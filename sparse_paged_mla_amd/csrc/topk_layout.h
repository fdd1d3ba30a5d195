// Layout of the caller-owned top-k workspace (host-side arithmetic only, so
// that the C-ABI validation layer can size it without any device code).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <algorithm>

namespace spmla {

constexpr int kTkThreads = 256;
constexpr int kTkPer = 32;                       // keys per thread per chunk
constexpr int kTkChunk = kTkThreads * kTkPer;    // 8192 keys per collect workgroup
constexpr int kTkSlice = 2048;                   // candidate slots per chunk
constexpr size_t kTopkScratchBytes = (size_t)32 << 20;  // static workspace of topk_select_noalloc
constexpr int kMaxDevices = 64;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline int32_t n_chunks(int64_t max_len) {
  return (int32_t)std::max<int64_t>(1, (max_len + kTkChunk - 1) / kTkChunk);
}

// Per request 8 bytes (its published threshold); per (request, chunk) 16
// bytes of metadata and a kTkSlice-entry (score bits, index) slice of
// candidates.
inline size_t topk_workspace_size(int32_t batch, int64_t max_len, int32_t k) {
  (void)k;
  if (batch <= 0 || max_len < 0) return 0;
  const size_t bc = (size_t)batch * (size_t)n_chunks(max_len);
  return align_up((size_t)batch * 8, 256) + align_up(bc * 16, 256) + bc * kTkSlice * 8;
}

}  // namespace spmla
