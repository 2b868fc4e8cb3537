// Anchor gather and varlen packing ("SuffixReplay", Algorithm Design 2:
// anchors live on 64-token pages; System Design, Pipelined Replay Path:
// several hits are packed into one variable-length batch with device-side
// boundaries).
//
// Kernel 1 (one workgroup) writes cu = exclusive prefix sum of the replay
// lengths.  Kernel 2 copies one packed row per wave with 16-byte vector
// loads/stores: packed row r belongs to the request i with cu[i] <= r <
// cu[i+1] (binary search), prefix position p = m_i - k_i + (r - cu[i]),
// source page page_table[i][p / 64], row p % 64.  Page ids and page-table
// columns are clamped into range so a corrupt table cannot read outside the
// pool (the copied data is then meaningless, but the launch stays in bounds).
#include <stdint.h>

#include "sr_common.hpp"
#include "sr_internal.hpp"

namespace sr {
namespace {

constexpr int kPage = 64;

__global__ __launch_bounds__(1024) void suffix_cu_kernel(const int32_t* __restrict__ k,
                                                          int n, int32_t* __restrict__ cu) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const int lane = tid % kWave, wv = tid / kWave;
  if (tid == 0) {
    carry = 0;
    cu[0] = 0;
  }
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + tid;
    int x = i < n ? max(k[i], 0) : 0;
    // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off, kWave);
      if (lane >= off) x += y;
    }
    if (lane == kWave - 1) wsum[wv] = x;
    __syncthreads();
    int pre = 0;
    for (int q = 0; q < wv; ++q) pre += wsum[q];
    const int c = carry;
    if (i < n) cu[i + 1] = c + pre + x;
    __syncthreads();
    if (tid == 1023) carry = c + pre + x;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(
    const uint8_t* __restrict__ pool, int64_t n_pages, int row_bytes,
    const int32_t* __restrict__ pt, int pt_stride, const int32_t* __restrict__ m_len,
    const int32_t* __restrict__ k_len, int n_req, const int32_t* __restrict__ cu,
    int total, uint8_t* __restrict__ out) {
  const int r = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (r >= total || r >= cu[n_req]) return;  // rows past sum(k) stay untouched
  // request owning row r: largest i with cu[i] <= r
  int lo = 0, hi = n_req - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int i = lo;
  int p = m_len[i] - k_len[i] + (r - cu[i]);
  p = max(p, 0);
  const int col = min(p / kPage, pt_stride - 1);
  int64_t page = pt[static_cast<int64_t>(i) * pt_stride + col];
  page = page < 0 ? 0 : (page >= n_pages ? n_pages - 1 : page);
  const uint8_t* src = pool + (page * kPage + (p % kPage)) * static_cast<int64_t>(row_bytes);
  uint8_t* dst = out + static_cast<int64_t>(r) * row_bytes;
  const int nvec = row_bytes / 16;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  for (int e = lane; e < nvec; e += kWave)
    reinterpret_cast<u32x4*>(dst)[e] = reinterpret_cast<const u32x4*>(src)[e];
}

}  // namespace
}  // namespace sr

extern "C" int sr_gather_suffix(const void* pool, int32_t hidden, int32_t elem_bytes,
                                int64_t n_pages, const int32_t* page_table,
                                int32_t pt_stride, const int32_t* matched_len,
                                const int32_t* suffix_len, int32_t n_req,
                                int32_t total_tokens, void* packed,
                                int32_t* cu_seqlens_out, void* stream) {
  if (n_req < 0 || total_tokens < 0 || hidden < 1 || pt_stride < 1) return SR_ESHAPE;
  if (elem_bytes != 2 && elem_bytes != 4) return SR_EDTYPE;
  const int64_t row_bytes = static_cast<int64_t>(hidden) * elem_bytes;
  if (row_bytes % 16 != 0 || row_bytes > INT32_MAX) return SR_ESHAPE;
  if (!cu_seqlens_out) return SR_EINVAL;
  if (n_req > 0 && (!matched_len || !suffix_len)) return SR_EINVAL;
  if (total_tokens > 0 && (n_req == 0 || !pool || !page_table || !packed || n_pages < 1))
    return n_req == 0 ? SR_ESHAPE : SR_EINVAL;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (total_tokens > 0 && (!al16(pool) || !al16(packed))) return SR_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(sr::suffix_cu_kernel, dim3(1), dim3(1024), 0, s, suffix_len, n_req,
                     cu_seqlens_out);
  if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
  if (total_tokens > 0) {
    const int blocks = (total_tokens + 3) / 4;
    hipLaunchKernelGGL(sr::gather_rows_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(pool), n_pages, static_cast<int>(row_bytes),
                       page_table, pt_stride, matched_len, suffix_len, n_req,
                       cu_seqlens_out, total_tokens, static_cast<uint8_t*>(packed));
    if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
  }
  return SR_OK;
}
