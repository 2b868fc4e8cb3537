// Token-serial gated-delta-rule replay in fp32 ("SuffixReplay", Eq. 4 with a
// decay plus rank-one erase; "Tail-Replay", section 2).
//
// One workgroup per (sequence, value head); the d_v x d_k state lives in
// registers, TPR threads per state row.  Used for fp32 inputs, where the
// fp16 matrix-core operands of the chunked kernel would cost precision, and
// for head sizes the chunked kernel does not cover.  Per token:
//   erase:      x = S k;  S <- a S + b (v - a x) k^T
//   erase-free: S <- a S + (b v) k^T
//   o = scale * S q
#include "sr_common.hpp"
#include "sr_internal.hpp"

namespace sr {

namespace {

constexpr int kSerialThreads = 256;
constexpr int kSerialTok = 32;  // tokens staged in LDS per step

template <int DK, int DV, typename TI, typename TO, bool ERASE>
__global__ __launch_bounds__(kSerialThreads) void gdn_serial_kernel(GdnArgs a) {
  constexpr int TPR = kSerialThreads / DV;  // threads per state row
  constexpr int JPT = DK / TPR;             // state columns per thread
  static_assert(TPR >= 1 && DK % TPR == 0, "bad tiling");
  __shared__ float sk[kSerialTok][DK];
  __shared__ float sq[kSerialTok][DK];
  __shared__ float sv[kSerialTok][DV];
  __shared__ float sa[kSerialTok];
  __shared__ float sb[kSerialTok];

  const int n = blockIdx.x / a.h_v;
  const int h = blockIdx.x % a.h_v;
  const int g = h / (a.h_v / a.h_k);
  const int tid = threadIdx.x;
  const int row = tid / TPR;
  const int j0 = (tid % TPR) * JPT;
  const bool want_o = a.o != nullptr;

  float S[JPT];
  const size_t sbase = (static_cast<size_t>(n) * a.h_v + h) * DK * DV;
#pragma unroll
  for (int e = 0; e < JPT; ++e)
    S[e] = a.s0 ? a.s0[sbase + static_cast<size_t>(j0 + e) * DV + row] : 0.0f;

  const int t_begin = a.cu[n];
  const int t_end = a.cu[n + 1];
  for (int c0 = t_begin; c0 < t_end; c0 += kSerialTok) {
    const int nv = min(kSerialTok, t_end - c0);
    __syncthreads();
    for (int e = tid; e < kSerialTok * DK; e += kSerialThreads) {
      const int t = e / DK, j = e % DK;
      const bool ok = t < nv;
      const size_t gi = (static_cast<size_t>(c0 + t) * a.h_k + g) * DK + j;
      sk[t][j] = ok ? load1<TI>(a.k, gi) : 0.0f;
      sq[t][j] = (ok && want_o) ? load1<TI>(a.q, gi) : 0.0f;
    }
    for (int e = tid; e < kSerialTok * DV; e += kSerialThreads) {
      const int t = e / DV, i = e % DV;
      sv[t][i] = t < nv ? load1<TI>(a.v, (static_cast<size_t>(c0 + t) * a.h_v + h) * DV + i)
                        : 0.0f;
    }
    if (tid < kSerialTok) {
      const bool ok = tid < nv;
      const size_t gi = static_cast<size_t>(c0 + tid) * a.h_v + h;
      float al = ok ? a.alpha[gi] : 1.0f;
      if (ok && a.alpha_is_log) al = expf(fmaxf(al, -64.0f));
      sa[tid] = al;
      sb[tid] = ok ? (a.beta ? a.beta[gi] : 1.0f) : 0.0f;
    }
    __syncthreads();
    for (int t = 0; t < nv; ++t) {
      const float al = sa[t];
      const float be = sb[t];
      float w;  // coefficient of k^T in the rank-one write
      if (ERASE) {
        float x = 0.0f;
#pragma unroll
        for (int e = 0; e < JPT; ++e) x = fmaf(S[e], sk[t][j0 + e], x);
#pragma unroll
        for (int off = TPR / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
        w = be * (sv[t][row] - al * x);
      } else {
        w = be * sv[t][row];
      }
#pragma unroll
      for (int e = 0; e < JPT; ++e) S[e] = fmaf(al, S[e], w * sk[t][j0 + e]);
      if (want_o) {
        float o = 0.0f;
#pragma unroll
        for (int e = 0; e < JPT; ++e) o = fmaf(S[e], sq[t][j0 + e], o);
#pragma unroll
        for (int off = TPR / 2; off >= 1; off >>= 1) o += __shfl_xor(o, off, kWave);
        if ((tid % TPR) == 0)
          store1<TO>(a.o, (static_cast<size_t>(c0 + t) * a.h_v + h) * DV + row, a.scale * o);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < JPT; ++e) a.s_out[sbase + static_cast<size_t>(j0 + e) * DV + row] = S[e];
}

template <int DK, int DV, typename TI, typename TO>
hipError_t launch_dkdv(const GdnArgs& a, hipStream_t s) {
  dim3 grid(a.n_seqs * a.h_v), block(kSerialThreads);
  if (a.erase)
    hipLaunchKernelGGL((gdn_serial_kernel<DK, DV, TI, TO, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gdn_serial_kernel<DK, DV, TI, TO, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <typename TI, typename TO>
hipError_t launch_ti_to(const GdnArgs& a, hipStream_t s) {
#define SR_DK_DV(dk, dv) \
  if (a.d_k == dk && a.d_v == dv) return launch_dkdv<dk, dv, TI, TO>(a, s);
  SR_DK_DV(32, 32) SR_DK_DV(32, 64) SR_DK_DV(32, 128)
  SR_DK_DV(64, 32) SR_DK_DV(64, 64) SR_DK_DV(64, 128)
  SR_DK_DV(128, 32) SR_DK_DV(128, 64) SR_DK_DV(128, 128)
#undef SR_DK_DV
  return hipErrorInvalidValue;
}

template <typename TI>
hipError_t launch_ti(const GdnArgs& a, hipStream_t s) {
  switch (a.dtype_o) {
    case SR_BF16: return launch_ti_to<TI, BF16>(a, s);
    case SR_F16: return launch_ti_to<TI, F16>(a, s);
    default: return launch_ti_to<TI, F32>(a, s);
  }
}

}  // namespace

bool gdn_serial_supports(int d_k, int d_v) {
  auto ok = [](int d) { return d == 32 || d == 64 || d == 128; };
  return ok(d_k) && ok(d_v);
}

hipError_t launch_gdn_serial(const GdnArgs& a, hipStream_t s) {
  if (a.n_seqs == 0) return hipSuccess;
  switch (a.dtype_qkv) {
    case SR_BF16: return launch_ti<BF16>(a, s);
    case SR_F16: return launch_ti<F16>(a, s);
    default: return launch_ti<F32>(a, s);
  }
}

}  // namespace sr
