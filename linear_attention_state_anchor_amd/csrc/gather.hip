// Anchor gather and varlen packing ("SuffixReplay", Algorithm Design 2:
// anchors on 64-token pages, optionally kept at only a subset of positions;
// Algorithm Design 3: the replay length counts anchors; System Design,
// Pipelined Replay Path: several hits are packed into one variable-length
// batch with device-side boundaries).
//
// Every 64-token page p of a prefix owns an anchor block of A rows; row j
// holds the anchor at position 64 p + off[j] (A = 64, off = 0..63: every
// token is an anchor).  Request i with matched length m_i has
// n_i = A floor(m_i / 64) + #{j : off[j] < m_i mod 64} anchors, in position
// order; its replay is the last k_i of them.
//
// Kernel 1 (one workgroup) writes cu = exclusive prefix sum of the replay
// lengths.  Kernel 2 copies one packed row per wave with 16-byte vector
// loads/stores: packed row r belongs to the request i with cu[i] <= r <
// cu[i+1] (binary search), anchor a = n_i - k_i + (r - cu[i]), source block
// page_table[i][a / A], row a % A.  Page ids and page-table columns are
// clamped into range so a corrupt table cannot read outside the pool (the
// copied data is then meaningless, but the launch stays in bounds).
#include <stdint.h>
#include <math.h>

#include <algorithm>

#include "sr_common.hpp"
#include "sr_internal.hpp"

namespace sr {
namespace {

constexpr int kPage = 64;

struct AnchorLayout {
  int a;        // anchor rows per page (1..64)
  int dense;    // 1: a = 64 and off[j] = j
  int off[64];  // in-page positions, strictly increasing
};

__device__ __forceinline__ int64_t anchors_in(int64_t m, const AnchorLayout& L) {
  if (L.dense) return m;
  int64_t n = (m / kPage) * L.a;
  const int rem = static_cast<int>(m % kPage);
  for (int j = 0; j < L.a; ++j) n += L.off[j] < rem;
  return n;
}

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

__device__ __forceinline__ void copy_row(int r, int lane, const uint8_t* __restrict__ pool,
                                         int64_t n_blocks, int row_bytes, const AnchorLayout& lay,
                                         const int32_t* __restrict__ pt, int pt_stride,
                                         const int32_t* __restrict__ m_len,
                                         const int32_t* __restrict__ k_len, int n_req,
                                         const int32_t* __restrict__ cu, uint8_t* __restrict__ out,
                                         int32_t* __restrict__ positions);

// One wave per packed row, grid-stride over the rows (the launch bounds the
// grid: a gather from host memory is bound by the host link and only needs
// a few CUs, which leaves the rest to work on other streams).
__global__ __launch_bounds__(256) void gather_rows_kernel(
    const uint8_t* __restrict__ pool, int64_t n_blocks, int row_bytes, AnchorLayout lay,
    const int32_t* __restrict__ pt, int pt_stride, const int32_t* __restrict__ m_len,
    const int32_t* __restrict__ k_len, int n_req, const int32_t* __restrict__ cu,
    int total, uint8_t* __restrict__ out, int32_t* __restrict__ positions) {
  const int lane = threadIdx.x % kWave;
  const int rows = min(total, cu[n_req]);  // rows past sum(k) stay untouched
  for (int r = blockIdx.x * 4 + threadIdx.x / kWave; r < rows; r += gridDim.x * 4)
    copy_row(r, lane, pool, n_blocks, row_bytes, lay, pt, pt_stride, m_len, k_len, n_req, cu,
             out, positions);
}

// Packed row r (one wave): find its request, anchor, block and row, copy it.
__device__ __forceinline__ void copy_row(int r, int lane, const uint8_t* __restrict__ pool,
                                         int64_t n_blocks, int row_bytes, const AnchorLayout& lay,
                                         const int32_t* __restrict__ pt, int pt_stride,
                                         const int32_t* __restrict__ m_len,
                                         const int32_t* __restrict__ k_len, int n_req,
                                         const int32_t* __restrict__ cu, uint8_t* __restrict__ out,
                                         int32_t* __restrict__ positions) {
  // request owning row r: largest i with cu[i] <= r
  int lo = 0, hi = n_req - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int i = lo;
  int64_t a = anchors_in(m_len[i], lay) - k_len[i] + (r - cu[i]);
  a = a < 0 ? 0 : a;
  const int64_t pcol = a / lay.a;
  const int j = static_cast<int>(a % lay.a);
  const int col = static_cast<int>(pcol < pt_stride - 1 ? pcol : pt_stride - 1);
  int64_t page = pt[static_cast<int64_t>(i) * pt_stride + col];
  page = page < 0 ? 0 : (page >= n_blocks ? n_blocks - 1 : page);
  const uint8_t* src = pool + (page * lay.a + j) * static_cast<int64_t>(row_bytes);
  uint8_t* dst = out + static_cast<int64_t>(r) * row_bytes;
  const int nvec = row_bytes / 16;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  for (int e = lane; e < nvec; e += kWave)
    reinterpret_cast<u32x4*>(dst)[e] = reinterpret_cast<const u32x4*>(src)[e];
  if (positions && lane == 0)
    positions[r] = static_cast<int32_t>(pcol * kPage + (lay.dense ? j : lay.off[j]));
}

int gather(const void* pool, int32_t hidden, int32_t elem_bytes, int64_t n_blocks,
           int32_t anchors_per_page, const int32_t* page_offsets, const int32_t* page_table,
           int32_t pt_stride, const int32_t* matched_len, const int32_t* suffix_len,
           int32_t n_req, int32_t total_tokens, void* packed, int32_t* cu_seqlens_out,
           int32_t* positions_out, void* stream) {
  if (n_req < 0 || total_tokens < 0 || hidden < 1 || pt_stride < 1) return SR_ESHAPE;
  if (elem_bytes != 2 && elem_bytes != 4) return SR_EDTYPE;
  if (anchors_per_page < 1 || anchors_per_page > kPage) return SR_ESHAPE;
  AnchorLayout lay{};
  lay.a = anchors_per_page;
  lay.dense = page_offsets == nullptr && anchors_per_page == kPage;
  if (!page_offsets && !lay.dense) return SR_EINVAL;
  for (int j = 0; j < lay.a; ++j) {
    lay.off[j] = page_offsets ? page_offsets[j] : j;
    if (lay.off[j] < 0 || lay.off[j] >= kPage || (j > 0 && lay.off[j] <= lay.off[j - 1]))
      return SR_ESHAPE;
  }
  if (lay.a == kPage) lay.dense = 1;  // offsets 0..63 are the only increasing choice
  const int64_t row_bytes = static_cast<int64_t>(hidden) * elem_bytes;
  if (row_bytes % 16 != 0 || row_bytes > INT32_MAX) return SR_ESHAPE;
  if (!cu_seqlens_out) return SR_EINVAL;
  if (n_req > 0 && (!matched_len || !suffix_len)) return SR_EINVAL;
  if (total_tokens > 0 && (n_req == 0 || !pool || !page_table || !packed || n_blocks < 1))
    return n_req == 0 ? SR_ESHAPE : SR_EINVAL;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (total_tokens > 0 && (!al16(pool) || !al16(packed))) return SR_EINVAL;
  // A pool in pinned host memory is read through its device mapping; memory
  // the runtime does not know (pageable host memory) is rejected.
  const void* dev_pool = pool;
  bool dev_host = false;  // the pool is host memory read through a mapping
  if (total_tokens > 0) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, pool) != hipSuccess) {
      (void)hipGetLastError();
      return SR_EINVAL;
    }
    if (attr.type == hipMemoryTypeUnregistered) return SR_EINVAL;
    if (attr.type == hipMemoryTypeHost) {
      if (!attr.devicePointer || !al16(attr.devicePointer)) return SR_EINVAL;
      dev_pool = attr.devicePointer;
      dev_host = true;
    }
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_checks_enabled()) {
    const int c = check_gather(n_blocks, lay.a, lay.off, page_table, pt_stride, matched_len,
                               suffix_len, n_req, total_tokens, s);
    if (c != SR_OK) return c;
  }
  hipLaunchKernelGGL(suffix_cu_kernel, dim3(1), dim3(1024), 0, s, suffix_len, n_req,
                     cu_seqlens_out);
  if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
  if (total_tokens > 0) {
    // device pool: enough workgroups to fill the chip; host pool: a few
    const int cap = dev_host ? 64 : 4096;
    const int blocks = std::min((total_tokens + 3) / 4, cap);
    hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint8_t*>(dev_pool), n_blocks, static_cast<int>(row_bytes),
                       lay, page_table, pt_stride, matched_len, suffix_len, n_req,
                       cu_seqlens_out, total_tokens, static_cast<uint8_t*>(packed),
                       positions_out);
    if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
  }
  return SR_OK;
}

}  // namespace
}  // namespace sr

extern "C" int sr_gather_suffix(const void* pool, int32_t hidden, int32_t elem_bytes,
                                int64_t n_pages, const int32_t* page_table,
                                int32_t pt_stride, const int32_t* matched_len,
                                const int32_t* suffix_len, int32_t n_req,
                                int32_t total_tokens, void* packed,
                                int32_t* cu_seqlens_out, void* stream) {
  return sr::gather(pool, hidden, elem_bytes, n_pages, sr::kPage, nullptr, page_table, pt_stride,
                    matched_len, suffix_len, n_req, total_tokens, packed, cu_seqlens_out,
                    nullptr, stream);
}

extern "C" int sr_gather_anchors(const void* pool, int32_t hidden, int32_t elem_bytes,
                                 int64_t n_blocks, int32_t anchors_per_page,
                                 const int32_t* page_offsets, const int32_t* page_table,
                                 int32_t pt_stride, const int32_t* matched_len,
                                 const int32_t* suffix_len, int32_t n_req,
                                 int32_t total_tokens, void* packed,
                                 int32_t* cu_seqlens_out, int32_t* positions_out,
                                 void* stream) {
  if (!page_offsets) return SR_EINVAL;
  return sr::gather(pool, hidden, elem_bytes, n_blocks, anchors_per_page, page_offsets,
                    page_table, pt_stride, matched_len, suffix_len, n_req, total_tokens, packed,
                    cu_seqlens_out, positions_out, stream);
}

extern "C" int64_t sr_replay_budget(const int32_t* n_anchors, int32_t n_req, double ratio,
                                    int32_t k_max, int32_t* k) {
  if (n_req < 0 || !(ratio > 0.0 && ratio <= 1.0)) return -1;
  if (n_req > 0 && (!n_anchors || !k)) return -1;
  int64_t sum = 0;
  for (int32_t i = 0; i < n_req; ++i) {
    const int32_t n = n_anchors[i];
    if (n < 0) return -1;
    // ceil(ratio * n) of the decimal ratio: a product within 1e-9 above an
    // integer counts as that integer (0.05 or 0.07 are not exact in binary,
    // and e.g. 0.07 * 100 evaluates to 7.000000000000001)
    const double x = ratio * static_cast<double>(n);
    const double fl = floor(x);
    int64_t want = static_cast<int64_t>(x - fl <= 1e-9 ? fl : fl + 1.0);
    if (want > n) want = n;
    if (k_max > 0 && want > k_max) want = k_max;
    k[i] = static_cast<int32_t>(want);
    sum += want;
  }
  return sum;
}
