// Single-token decode step of the gated delta rule, continuing from a
// reconstructed state ("Tail-Replay", section 3: the unmatched tokens
// continue from the reconstructed linear-attention states; "SuffixReplay",
// Eq. 4 applied to one more token).
//
// Per sequence n (one token each) and value head h, with S^T stored
// [d_k][d_v] (row j = key, column i = value):
//     x   = S k                                  x_i = sum_j S^T[j][i] k_j
//     S'  = a S (I - b k k^T) + b v k^T          S'^T[j][i] = a S^T[j][i] + k_j u_i,
//                                                 u_i = b (v_i - a x_i)
//     o   = scale S' q                           o_i = scale sum_j S'^T[j][i] q_j
// (erase-free: u_i = b v_i).  One workgroup of 4 waves per (sequence, head):
// wave w holds key rows [w d_k/4, (w+1) d_k/4) of S^T in registers, a lane
// D/64 adjacent value columns, so the state is read once and written once
// with coalesced row accesses; the two sums over keys are wave partial sums
// combined through LDS.  HBM-bound: 2 d_k d_v fp32 per (sequence, head).
#include <stdint.h>

#include "sr_common.hpp"
#include "sr_internal.hpp"

namespace sr {
namespace {

constexpr int kDecWaves = 4;

template <typename T>
__device__ __forceinline__ float ld1(const void* p, size_t i) {
  return load1<T>(p, i);
}

template <int D, typename TI, typename TO, bool ERASE>
__global__ __launch_bounds__(64 * kDecWaves) void gdn_decode_kernel(GdnArgs a) {
  constexpr int CPL = D / kWave;        // value columns per lane
  constexpr int RPW = D / kDecWaves;    // key rows per wave
  __shared__ float part[kDecWaves][D];  // per-wave partial sums over keys
  __shared__ float u_sh[D];
  const int n = blockIdx.x / a.h_v;
  const int h = blockIdx.x % a.h_v;
  const int g = h / (a.h_v / a.h_k);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int lane = threadIdx.x % kWave;
  const int i0 = CPL * lane;            // first value column of this lane
  const int j0 = w * RPW;               // first key row of this wave
  const size_t sbase = (static_cast<size_t>(n) * a.h_v + h) * D * D;
  const size_t kq = (static_cast<size_t>(n) * a.h_k + g) * D;
  const size_t vb = (static_cast<size_t>(n) * a.h_v + h) * D;
  const float al = a.alpha_is_log ? __expf(fmaxf(a.alpha[static_cast<size_t>(n) * a.h_v + h], -64.0f))
                                  : a.alpha[static_cast<size_t>(n) * a.h_v + h];
  const float be = a.beta ? a.beta[static_cast<size_t>(n) * a.h_v + h] : 1.0f;

  // CPL adjacent fp32 columns per lane and row: one 8-byte (d = 128) or
  // 4-byte (d = 64) access, a wave covering one contiguous row
  typedef float fv __attribute__((ext_vector_type(CPL)));
  float s[RPW][CPL];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const fv x = a.s0 ? *reinterpret_cast<const fv*>(a.s0 + sbase + static_cast<size_t>(j0 + r) * D + i0)
                      : fv{};
#pragma unroll
    for (int e = 0; e < CPL; ++e) s[r][e] = x[e];
  }
  float kr[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) kr[r] = ld1<TI>(a.k, kq + j0 + r);

  float u[CPL];
  if (ERASE) {
    // x_i partial over this wave's keys, combined across the waves in LDS
    float x[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      x[e] = 0.0f;
#pragma unroll
      for (int r = 0; r < RPW; ++r) x[e] = fmaf(s[r][e], kr[r], x[e]);
      part[w][i0 + e] = x[e];
    }
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        float xs = 0.0f;
#pragma unroll
        for (int q = 0; q < kDecWaves; ++q) xs += part[q][i0 + e];
        u_sh[i0 + e] = be * (ld1<TI>(a.v, vb + i0 + e) - al * xs);
      }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < CPL; ++e) u[e] = u_sh[i0 + e];
  } else {
#pragma unroll
    for (int e = 0; e < CPL; ++e) u[e] = be * ld1<TI>(a.v, vb + i0 + e);
  }

  // S'^T = a S^T + k u^T, stored; o partial sums over this wave's keys
  const bool want_o = a.o != nullptr;
  float o[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) o[e] = 0.0f;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const float qj = want_o ? ld1<TI>(a.q, kq + j0 + r) : 0.0f;
    fv x;
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      s[r][e] = fmaf(kr[r], u[e], al * s[r][e]);
      x[e] = s[r][e];
      o[e] = fmaf(s[r][e], qj, o[e]);
    }
    *reinterpret_cast<fv*>(a.s_out + sbase + static_cast<size_t>(j0 + r) * D + i0) = x;
  }
  if (!want_o) return;
  __syncthreads();  // part[] is reused
#pragma unroll
  for (int e = 0; e < CPL; ++e) part[w][i0 + e] = o[e];
  __syncthreads();
  if (w == 0) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      float os = 0.0f;
#pragma unroll
      for (int q = 0; q < kDecWaves; ++q) os += part[q][i0 + e];
      store1<TO>(a.o, vb + i0 + e, a.scale * os);
    }
  }
}

template <int D, typename TI, typename TO>
hipError_t launch_dec3(const GdnArgs& a, hipStream_t s) {
  const dim3 grid(a.n_seqs * a.h_v), block(64 * kDecWaves);
  if (a.erase)
    hipLaunchKernelGGL((gdn_decode_kernel<D, TI, TO, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gdn_decode_kernel<D, TI, TO, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D, typename TI>
hipError_t launch_dec2(const GdnArgs& a, hipStream_t s) {
  switch (a.dtype_o) {
    case SR_BF16: return launch_dec3<D, TI, BF16>(a, s);
    case SR_F16: return launch_dec3<D, TI, F16>(a, s);
    default: return launch_dec3<D, TI, F32>(a, s);
  }
}

template <int D>
hipError_t launch_dec1(const GdnArgs& a, hipStream_t s) {
  switch (a.dtype_qkv) {
    case SR_BF16: return launch_dec2<D, BF16>(a, s);
    case SR_F16: return launch_dec2<D, F16>(a, s);
    default: return launch_dec2<D, F32>(a, s);
  }
}

}  // namespace
}  // namespace sr

extern "C" int sr_gdn_decode_step(const sr_gdn_desc* d, const sr_gdn_io* io, void* stream) {
  if (!d || !io) return SR_EINVAL;
  if (d->n_seqs < 0 || d->total_tokens != d->n_seqs || d->h_k < 1 || d->h_v < 1 ||
      d->h_v % d->h_k != 0 || d->d_k != d->d_v || (d->d_k != 64 && d->d_k != 128))
    return SR_ESHAPE;
  auto dt_ok = [](int t) { return t == SR_BF16 || t == SR_F16 || t == SR_F32; };
  if (!dt_ok(d->dtype_qkv) || !dt_ok(d->dtype_o)) return SR_EDTYPE;
  if ((d->erase != 0 && d->erase != 1) || (d->alpha_is_log != 0 && d->alpha_is_log != 1))
    return SR_EINVAL;
  if (d->n_seqs == 0) return SR_OK;
  if (static_cast<int64_t>(d->n_seqs) * d->h_v > INT32_MAX) return SR_ESHAPE;
  if (!io->k || !io->v || !io->alpha || !io->final_state) return SR_EINVAL;
  if (io->o && !io->q) return SR_EINVAL;
  // states are accessed 8 bytes at a time (d = 128)
  auto al8 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; };
  if (!al8(io->final_state) || (io->initial_state && !al8(io->initial_state))) return SR_EINVAL;
  sr::GdnArgs a{};
  a.n_seqs = d->n_seqs;
  a.total_tokens = d->total_tokens;
  a.h_k = d->h_k;
  a.h_v = d->h_v;
  a.d_k = d->d_k;
  a.d_v = d->d_v;
  a.dtype_qkv = d->dtype_qkv;
  a.dtype_o = d->dtype_o;
  a.erase = d->erase;
  a.alpha_is_log = d->alpha_is_log;
  a.scale = d->scale;
  a.q = io->q;
  a.k = io->k;
  a.v = io->v;
  a.alpha = io->alpha;
  a.beta = io->beta;
  a.cu = nullptr;
  a.s0 = io->initial_state;
  a.s_out = io->final_state;
  a.o = io->o;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = d->d_k == 128 ? sr::launch_dec1<128>(a, s) : sr::launch_dec1<64>(a, s);
  return e == hipSuccess ? SR_OK : SR_ELAUNCH;
}
