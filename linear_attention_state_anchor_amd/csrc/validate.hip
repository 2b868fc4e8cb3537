// Validation of the preconditions that live in device memory ("SuffixReplay",
// System Design, Pipelined Replay Path: hits are packed into one
// variable-length execution with device-side boundaries, which these checks
// validate; Eq. 4 / "Tail-Replay" section 2: the gate alpha lies in (0, 1]).
//
// The release path never reads device data on the host.  The checks here run
// only on request (sr_check_* or the SR_DEBUG=1 environment variable): a
// kernel sets bits of a small per-device result array, and the host waits
// for it and reads the bits back.  The result array is a file-scope device
// symbol; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device.  Checks on one device are serialised by a
// host mutex.
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "sr_common.hpp"
#include "sr_internal.hpp"

namespace sr {
namespace {

// [0]: violation bits, [1..2]: 64-bit sum of replay lengths
__device__ __align__(16) unsigned int g_check[4];

constexpr unsigned kBadCu = 1u, kBadAlpha = 2u, kBadBeta = 4u, kBadLens = 8u, kBadPage = 16u;

__global__ void check_zero_kernel(unsigned int* r) {
  if (threadIdx.x < 4) r[threadIdx.x] = 0u;
}

__global__ void check_cu_kernel(const int32_t* __restrict__ cu, int n, int total,
                                unsigned int* r) {
  const int stride = gridDim.x * blockDim.x;
  bool bad = false;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    bad |= cu[i + 1] < cu[i];
  if (blockIdx.x == 0 && threadIdx.x == 0) bad |= cu[0] != 0 || cu[n] != total;
  if (bad) atomicOr(r, kBadCu);
}

__global__ void check_gates_kernel(const float* __restrict__ alpha, int alpha_is_log,
                                   const float* __restrict__ beta, size_t count,
                                   unsigned int* r) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  unsigned bits = 0u;
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < count;
       e += stride) {
    const float a = alpha[e];
    // written so that NaN fails every test
    const bool a_ok = alpha_is_log ? (a <= 0.0f) : (a > 0.0f && a <= 1.0f);
    if (!a_ok) bits |= kBadAlpha;
    if (beta) {
      const float b = beta[e];
      if (!(b >= 0.0f && b <= 2.0f)) bits |= kBadBeta;
    }
  }
  if (bits) atomicOr(r, bits);
}

struct Offsets {
  int a;        // anchors per page
  int off[64];  // in-page positions, increasing
};

// anchors of a prefix of m tokens
__device__ __forceinline__ int64_t anchors_of(int64_t m, const Offsets& o) {
  int64_t n = (m / 64) * o.a;
  const int rem = static_cast<int>(m % 64);
  for (int j = 0; j < o.a; ++j) n += o.off[j] < rem;
  return n;
}

__global__ void check_gather_kernel(Offsets o, int64_t n_blocks, const int32_t* __restrict__ pt,
                                    int pt_stride, const int32_t* __restrict__ m_len,
                                    const int32_t* __restrict__ k_len, int n_req,
                                    unsigned int* r) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_req) return;
  const int64_t m = m_len[i], k = k_len[i];
  unsigned bits = 0u;
  if (m < 0 || k < 0) {
    bits |= kBadLens;
  } else {
    const int64_t n = anchors_of(m, o);
    if (k > n) bits |= kBadLens;
    if (k > 0 && k <= n) {
      const int64_t c0 = (n - k) / o.a, c1 = (n - 1) / o.a;  // page-table columns read
      if (c1 >= pt_stride) {
        bits |= kBadPage;
      } else {
        for (int64_t c = c0; c <= c1; ++c) {
          const int64_t p = pt[static_cast<int64_t>(i) * pt_stride + c];
          if (p < 0 || p >= n_blocks) bits |= kBadPage;
        }
      }
    }
    atomicAdd(reinterpret_cast<unsigned long long*>(r + 2), static_cast<unsigned long long>(k));
  }
  if (bits) atomicOr(r, bits);
}

std::mutex g_check_mu;

// Address of this device's result array (looked up once per device).
hipError_t result_ptr(unsigned int** out) {
  static std::mutex mu;
  static unsigned int* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_check));
    if (e != hipSuccess) return e;
    ptrs[dev] = static_cast<unsigned int*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

// Runs `launch(result)` after clearing the result array, waits, and maps the
// violation bits (and, if want_sum >= 0, the length sum) to a status.
template <typename F>
int run_check(hipStream_t s, int64_t want_sum, F launch) {
  std::lock_guard<std::mutex> lk(g_check_mu);
  unsigned int* r = nullptr;
  if (result_ptr(&r) != hipSuccess) return SR_ELAUNCH;
  hipLaunchKernelGGL(check_zero_kernel, dim3(1), dim3(64), 0, s, r);
  if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
  if (!launch(r)) return SR_ELAUNCH;
  unsigned int host[4] = {};
  if (hipMemcpyAsync(host, r, sizeof(host), hipMemcpyDeviceToHost, s) != hipSuccess)
    return SR_ELAUNCH;
  if (hipStreamSynchronize(s) != hipSuccess) return SR_ELAUNCH;
  uint64_t sum = 0;
  memcpy(&sum, &host[2], sizeof(sum));
  if (host[0] != 0u) return SR_EDATA;
  if (want_sum >= 0 && sum != static_cast<uint64_t>(want_sum)) return SR_EDATA;
  return SR_OK;
}

bool launch_cu(hipStream_t s, const int32_t* cu, int n, int total, unsigned int* r) {
  const int blocks = std::max(1, std::min(256, (n + 255) / 256));
  hipLaunchKernelGGL(check_cu_kernel, dim3(blocks), dim3(256), 0, s, cu, n, total, r);
  return hipGetLastError() == hipSuccess;
}

}  // namespace

bool debug_checks_enabled() {
  const char* v = getenv("SR_DEBUG");
  return v && v[0] == '1' && v[1] == '\0';
}

int check_cu_seqlens(const int32_t* cu, int n_seqs, int total_tokens, hipStream_t s) {
  if (n_seqs < 0 || total_tokens < 0) return SR_ESHAPE;
  if (!cu) return SR_EINVAL;
  return run_check(s, -1, [&](unsigned int* r) { return launch_cu(s, cu, n_seqs, total_tokens, r); });
}

int check_replay(const GdnArgs& a, hipStream_t s) {
  return run_check(s, -1, [&](unsigned int* r) {
    if (!launch_cu(s, a.cu, a.n_seqs, a.total_tokens, r)) return false;
    const size_t count = static_cast<size_t>(a.total_tokens) * a.h_v;
    if (count == 0) return true;
    const int blocks = static_cast<int>(std::min<size_t>(1024, (count + 255) / 256));
    hipLaunchKernelGGL(check_gates_kernel, dim3(blocks), dim3(256), 0, s, a.alpha, a.alpha_is_log,
                       a.beta, count, r);
    return hipGetLastError() == hipSuccess;
  });
}

int check_gather(int64_t n_blocks, int anchors_per_page, const int32_t* offsets,
                 const int32_t* pt, int pt_stride, const int32_t* m_len,
                 const int32_t* k_len, int n_req, int total, hipStream_t s) {
  if (n_req < 0 || total < 0 || pt_stride < 1 || n_blocks < 0) return SR_ESHAPE;
  if (anchors_per_page < 1 || anchors_per_page > 64) return SR_ESHAPE;
  Offsets o{};
  o.a = anchors_per_page;
  for (int j = 0; j < o.a; ++j) {
    o.off[j] = offsets ? offsets[j] : j;
    if (o.off[j] < 0 || o.off[j] > 63 || (j > 0 && o.off[j] <= o.off[j - 1])) return SR_ESHAPE;
  }
  if (n_req == 0) return total == 0 ? SR_OK : SR_ESHAPE;
  if (!pt || !m_len || !k_len) return SR_EINVAL;
  return run_check(s, total, [&](unsigned int* r) {
    hipLaunchKernelGGL(check_gather_kernel, dim3((n_req + 255) / 256), dim3(256), 0, s, o,
                       n_blocks, pt, pt_stride, m_len, k_len, n_req, r);
    return hipGetLastError() == hipSuccess;
  });
}

}  // namespace sr

extern "C" int sr_check_gather_inputs(int64_t n_blocks, int32_t anchors_per_page,
                                      const int32_t* page_offsets, const int32_t* page_table,
                                      int32_t pt_stride, const int32_t* matched_len,
                                      const int32_t* suffix_len, int32_t n_req,
                                      int32_t total_tokens, void* stream) {
  return sr::check_gather(n_blocks, anchors_per_page, page_offsets, page_table, pt_stride,
                          matched_len, suffix_len, n_req, total_tokens,
                          static_cast<hipStream_t>(stream));
}
