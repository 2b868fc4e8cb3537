// Replay of one group of linear-attention layers from its entry anchors
// ("SuffixReplay", Algorithm Design 1: one anchor per group, only the linear
// layers run, full-attention layers are skipped; "Tail-Replay", section 3:
// zero initial state per group, the group's final FFN omitted).
//
// Per GDN layer (pre-norm residual block without FFN):
//   r_t  = (mean x_t^2 + eps)^(-1/2)                       rms_rows_kernel
//   P    = r o (x W_in), packed columns k|v|a|b|pad|q|z    gemm_kernel (MFMA)
//   q,k  = L2norm(SiLU(conv(P_q,P_k))), v = SiLU(conv(P_v)),
//   z, log a = -softplus(P_a), b = sigmoid(P_b)            frontend_kernel
//   S, o = gated delta rule from S_0 = 0                   launch_gdn_chunk
//   y    = rms(o) o SiLU(z) per value head                 gated_norm_kernel
//   x   <- x + y W_out                                     gemm_kernel (MFMA)
// The last GDN layer of the group only needs its state: its projection
// covers the k|v|a|b prefix of the packed columns (plus q when the conv
// windows are returned) and no output is formed.
#include <stdint.h>
#include <string.h>

#include <type_traits>

#include "sr_common.hpp"
#include "sr_internal.hpp"

namespace sr {
namespace {

constexpr size_t kAlign = 256;
__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// packed layer layout
// ---------------------------------------------------------------------------
struct LayerShape {
  int hidden, h_k, h_v, d, width;
  __host__ __device__ int n_kv() const { return (h_k + h_v) * d; }             // k|v columns
  __host__ __device__ int n_state() const { return n_kv() + 2 * h_v; }         // + a|b
  __host__ __device__ int n_state_pad() const { return static_cast<int>(align_up(n_state(), 128)); }
  __host__ __device__ int n_all() const { return static_cast<int>(align_up(n_state_pad() + (h_k + h_v) * d, 128)); }
  __host__ __device__ int q_off() const { return n_state_pad(); }              // q columns start
  __host__ __device__ int z_off() const { return n_state_pad() + h_k * d; }    // z columns start
  __host__ __device__ int a_off() const { return n_kv(); }
  __host__ __device__ int b_off() const { return n_kv() + h_v; }
  __host__ __device__ int conv_dim() const { return (2 * h_k + h_v) * d; }
  __host__ __device__ size_t win_bytes() const { return align_up(static_cast<size_t>(n_all()) * hidden * 2, kAlign); }
  __host__ __device__ size_t conv_bytes() const { return align_up(static_cast<size_t>(conv_dim()) * width * 4, kAlign); }
  __host__ __device__ size_t wout_bytes() const { return align_up(static_cast<size_t>(hidden) * h_v * d * 2, kAlign); }
  __host__ __device__ size_t total() const { return win_bytes() + conv_bytes() + wout_bytes(); }
  // packed column of an original input column (q|k|v|z|a|b order), or -1
  __host__ __device__ int packed_col(int c) const {
    const int nq = h_k * d, nv = h_v * d;
    if (c < nq) return n_state_pad() + c;                  // q
    c -= nq;
    if (c < nq) return c;                                  // k
    c -= nq;
    if (c < nv) return h_k * d + c;                        // v
    c -= nv;
    if (c < nv) return n_state_pad() + h_k * d + c;        // z
    c -= nv;
    if (c < 2 * h_v) return n_kv() + c;                    // a, b
    return -1;
  }
};

// conv channel index of packed column pc (k|v first, then q), or -1
__device__ __forceinline__ int conv_channel(const LayerShape& L, int pc) {
  if (pc < L.n_kv()) return pc;
  if (pc >= L.q_off() && pc < L.q_off() + L.h_k * L.d) return L.n_kv() + (pc - L.q_off());
  return -1;
}

// W_in bf16 [hidden][n_in] -> W_in^T fp16 [n_all][hidden] in packed column
// order (zero rows for padding).
__global__ void pack_win_kernel(const uint16_t* __restrict__ w, LayerShape L,
                                _Float16* __restrict__ wt) {
  const int n_in = 2 * L.h_k * L.d + 2 * L.h_v * L.d + 2 * L.h_v;
  const size_t total = static_cast<size_t>(L.n_all()) * L.hidden;
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<size_t>(gridDim.x) * blockDim.x)
    wt[e] = static_cast<_Float16>(0.0f);
  (void)n_in;
}
__global__ void pack_win_copy_kernel(const uint16_t* __restrict__ w, LayerShape L,
                                     _Float16* __restrict__ wt) {
  const int n_in = 2 * L.h_k * L.d + 2 * L.h_v * L.d + 2 * L.h_v;
  // one thread per (k, input column): reads are coalesced along columns
  const size_t total = static_cast<size_t>(L.hidden) * n_in;
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int k = static_cast<int>(e / n_in);
    const int c = static_cast<int>(e % n_in);
    const int pc = L.packed_col(c);
    wt[static_cast<size_t>(pc) * L.hidden + k] = static_cast<_Float16>(bf16_to_f32(w[e]));
  }
}
// conv bf16 [conv_dim][width] (q|k|v channels) -> fp32 in k|v|q channel order
__global__ void pack_conv_kernel(const uint16_t* __restrict__ cw, LayerShape L,
                                 float* __restrict__ out) {
  const int nq = L.h_k * L.d;
  const int total = L.conv_dim() * L.width;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
    const int c = e / L.width, j = e % L.width;
    int ch;  // channel in k|v|q order
    if (c < nq) ch = L.n_kv() + c;          // q
    else ch = c - nq;                       // k, v
    out[ch * L.width + j] = bf16_to_f32(cw[e]);
  }
}
// W_out bf16 [h_v d][hidden] -> W_out^T fp16 [hidden][h_v d]
__global__ void pack_wout_kernel(const uint16_t* __restrict__ w, LayerShape L,
                                 _Float16* __restrict__ wt) {
  const int K = L.h_v * L.d;
  const size_t total = static_cast<size_t>(K) * L.hidden;
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int k = static_cast<int>(e / L.hidden);
    const int n = static_cast<int>(e % L.hidden);
    wt[static_cast<size_t>(n) * K + k] = static_cast<_Float16>(bf16_to_f32(w[e]));
  }
}

// ---------------------------------------------------------------------------
// row statistics: r_t = (mean_c x_t,c^2 + eps)^(-1/2), one wave per row
// ---------------------------------------------------------------------------
template <typename TX>
__global__ __launch_bounds__(256) void rms_rows_kernel(const void* __restrict__ x, int rows,
                                                       int cols, float eps,
                                                       float* __restrict__ r) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  float s = 0.0f;
  for (int c = lane; c < cols; c += kWave) {
    const float v = load1<TX>(x, static_cast<size_t>(row) * cols + c);
    s = fmaf(v, v, s);
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
  if (lane == 0) r[row] = rsqrtf(s / static_cast<float>(cols) + eps);
}

// ---------------------------------------------------------------------------
// C[M][N] = epilogue(A[M][K] . Bt[N][K]^T), fp16 matrix-core operands
//   EPI_SCALE: C = rs[m] * acc                 (fp32 out)
//   EPI_RESID: C = X[m][n] + acc, X of type TX (fp32 out; C may alias X)
// Tile 128 x 128 x 64, 4 waves of 64 x 64, 32x32x16 MFMAs; the next k-tile
// is prefetched into registers while the current one is in LDS.
// Requirements: K % 64 == 0, N % 128 == 0, lda/ldb multiples of 8.
// ---------------------------------------------------------------------------
constexpr int EPI_SCALE = 0;
constexpr int EPI_RESID = 1;
constexpr int GBM = 128, GBN = 128, GBK = 64, GLD = GBK + 8;

template <typename TA>
struct ATile;
template <>
struct ATile<BF16> {  // 8 elements per 16-byte load
  static constexpr int kPer = 8;
};
template <>
struct ATile<F16> {
  static constexpr int kPer = 8;
};
template <>
struct ATile<F32> {  // 4 elements per 16-byte load
  static constexpr int kPer = 4;
};

template <typename TA, int EPI, typename TX>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const void* __restrict__ A, int lda,
                                                      const _Float16* __restrict__ Bt, int ldb,
                                                      int M, int N, int K, float* C, int ldc,
                                                      const float* __restrict__ rs,
                                                      const void* X, int ldx) {
  __shared__ _Float16 sa[GBM * GLD];
  __shared__ _Float16 sb[GBN * GLD];
  constexpr int PER = ATile<TA>::kPer;
  constexpr int A_LOADS = GBM * GBK / PER / 256;  // 16-byte loads per thread
  constexpr int B_LOADS = GBN * GBK / 8 / 256;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = tid % kWave;
  const int wm = w / 2, wn = w % 2;
  // tiles: blockIdx.x over N (fast), blockIdx.y over M
  const int n0 = blockIdx.x * GBN;
  const int m0 = blockIdx.y * GBM;

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 ra[A_LOADS], rb[B_LOADS];
  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
      const int item = tid + 256 * e;
      const int row = item / (GBK / PER), ch = item % (GBK / PER);
      const int m = m0 + row;
      ra[e] = u32x4{0u, 0u, 0u, 0u};
      if (m < M) {
        const char* p = static_cast<const char*>(A) +
                        (static_cast<size_t>(m) * lda + k0 + ch * PER) * sizeof(uint16_t) *
                            (PER == 4 ? 2 : 1);
        ra[e] = *reinterpret_cast<const u32x4*>(p);
      }
    }
#pragma unroll
    for (int e = 0; e < B_LOADS; ++e) {
      const int item = tid + 256 * e;
      const int row = item / (GBK / 8), ch = item % (GBK / 8);
      rb[e] = *reinterpret_cast<const u32x4*>(Bt + static_cast<size_t>(n0 + row) * ldb + k0 + ch * 8);
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int e = 0; e < A_LOADS; ++e) {
      const int item = tid + 256 * e;
      const int row = item / (GBK / PER), ch = item % (GBK / PER);
      if (PER == 8) {
        f16x8 v;
        if (std::is_same<TA, F16>::value) {
          v = __builtin_bit_cast(f16x8, ra[e]);
        } else {
          const u16x8 b = __builtin_bit_cast(u16x8, ra[e]);
#pragma unroll
          for (int x = 0; x < 8; ++x) v[x] = static_cast<_Float16>(bf16_to_f32(b[x]));
        }
        *reinterpret_cast<f16x8*>(&sa[row * GLD + ch * 8]) = v;
      } else {
        const f32x4 f = __builtin_bit_cast(f32x4, ra[e]);
        *reinterpret_cast<f16x4*>(&sa[row * GLD + ch * 4]) = to_f16x4(f);
      }
    }
#pragma unroll
    for (int e = 0; e < B_LOADS; ++e) {
      const int item = tid + 256 * e;
      const int row = item / (GBK / 8), ch = item % (GBK / 8);
      *reinterpret_cast<u32x4*>(&sb[row * GLD + ch * 8]) = rb[e];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  load_tiles(0);
  for (int k0 = 0; k0 < K; k0 += GBK) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (k0 + GBK < K) load_tiles(k0 + GBK);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      f16x8 av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *reinterpret_cast<const f16x8*>(
            &sa[(wm * 64 + 32 * i + l % 32) * GLD + ks * 16 + 8 * (l / 32)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bv[j] = *reinterpret_cast<const f16x8*>(
            &sb[(wn * 64 + 32 * j + l % 32) * GLD + ks * 16 + 8 * (l / 32)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(av[i], bv[j], acc[i][j]);
    }
  }
  // epilogue: lane holds column l%32 and rows 8(r/4) + 4(l/32) + r%4
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + 32 * i + 8 * (r / 4) + 4 * (l / 32) + (r % 4);
        const int n = n0 + wn * 64 + 32 * j + l % 32;
        if (m >= M || n >= N) continue;
        const size_t ci = static_cast<size_t>(m) * ldc + n;
        if (EPI == EPI_SCALE) {
          C[ci] = rs[m] * acc[i][j][r];
        } else {
          C[ci] = load1<TX>(X, static_cast<size_t>(m) * ldx + n) + acc[i][j][r];
        }
      }
}

// ---------------------------------------------------------------------------
// front-end epilogue, one workgroup per token, one wave per 128-channel head:
// causal conv (zero history before the sequence start) + SiLU on q|k|v,
// per-head L2 norm of q and k, z copy, gates.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void frontend_kernel(
    const float* __restrict__ P, int ldp, LayerShape L, const float* __restrict__ convw,
    const int32_t* __restrict__ seq_start, int T, float l2_eps, bool last,
    _Float16* __restrict__ qo, _Float16* __restrict__ ko, _Float16* __restrict__ vo,
    _Float16* __restrict__ zo, float* __restrict__ la, float* __restrict__ be) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const int s0 = seq_start[t];
  const int d = L.d;
  const int W = L.width;
  // heads: k (h_k), v (h_v), q (h_k, not for the last layer), z (h_v), gates
  const int nk = L.h_k, nv = L.h_v;
  const int n_heads = last ? nk + nv : 2 * nk + 2 * nv;
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int hh = wv; hh < n_heads; hh += blockDim.x / kWave) {
    int pc0, kind;  // kind 0: k, 1: v, 2: q, 3: z
    int hidx;
    if (hh < nk) { kind = 0; hidx = hh; pc0 = hh * d; }
    else if (hh < nk + nv) { kind = 1; hidx = hh - nk; pc0 = nk * d + hidx * d; }
    else if (hh < 2 * nk + nv) { kind = 2; hidx = hh - nk - nv; pc0 = L.q_off() + hidx * d; }
    else { kind = 3; hidx = hh - 2 * nk - nv; pc0 = L.z_off() + hidx * d; }
    float vals[4];
    int nvals = 0;
    float ss = 0.0f;
    for (int c = lane; c < d; c += kWave) {
      const int pc = pc0 + c;
      float y;
      if (kind == 3) {
        y = P[static_cast<size_t>(t) * ldp + pc];
      } else {
        const int ch = conv_channel(L, pc);
        float acc = 0.0f;
        for (int j = 0; j < W; ++j) {
          const int tt = t - (W - 1) + j;
          if (tt >= s0) acc = fmaf(convw[ch * W + j], P[static_cast<size_t>(tt) * ldp + pc], acc);
        }
        y = acc / (1.0f + __expf(-acc));  // SiLU
      }
      vals[nvals++] = y;
      ss = fmaf(y, y, ss);
    }
    if (kind == 0 || kind == 2) {
#pragma unroll
      for (int off = kWave / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
      const float inv = rsqrtf(ss + l2_eps);
      for (int e = 0; e < nvals; ++e) vals[e] *= inv;
    }
    _Float16* out = kind == 0 ? ko + (static_cast<size_t>(t) * nk + hidx) * d
                  : kind == 1 ? vo + (static_cast<size_t>(t) * nv + hidx) * d
                  : kind == 2 ? qo + (static_cast<size_t>(t) * nk + hidx) * d
                              : zo + (static_cast<size_t>(t) * nv + hidx) * d;
    int e = 0;
    for (int c = lane; c < d; c += kWave) out[c] = static_cast<_Float16>(vals[e++]);
  }
  // gates
  for (int h = threadIdx.x; h < nv; h += blockDim.x) {
    const float av = P[static_cast<size_t>(t) * ldp + L.a_off() + h];
    const float bv = P[static_cast<size_t>(t) * ldp + L.b_off() + h];
    la[static_cast<size_t>(t) * nv + h] = -softplus(av);
    be[static_cast<size_t>(t) * nv + h] = sigmoid(bv);
  }
}

// conv state: last W-1 pre-conv rows of q|k|v per sequence (original
// channel order), oldest first, zero where the sequence is shorter
__global__ void conv_state_kernel(const float* __restrict__ P, int ldp, LayerShape L,
                                  const int32_t* __restrict__ cu, int n_seqs,
                                  float* __restrict__ out) {
  const int n = blockIdx.y;
  const int W1 = L.width - 1;
  const int cd = L.conv_dim();
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < cd * W1; e += gridDim.x * blockDim.x) {
    const int c = e / W1, j = e % W1;
    const int start = cu[n], end = cu[n + 1];
    const int pos = end - W1 + j;
    float v = 0.0f;
    if (pos >= start) v = P[static_cast<size_t>(pos) * ldp + L.packed_col(c)];
    out[(static_cast<size_t>(n) * cd + c) * W1 + j] = v;
  }
}

__global__ void fill_kernel(float* __restrict__ p, size_t n, float v) {
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[e] = v;
}

// seq_start[t] = cu[n] for the sequence n holding token t
__global__ void seq_start_kernel(const int32_t* __restrict__ cu, int n_seqs, int T,
                                 int32_t* __restrict__ out) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  out[t] = cu[lo];
}

// y = o / sqrt(mean(o^2) + eps) * SiLU(z), per (token, value head), fp16 out
__global__ __launch_bounds__(256) void gated_norm_kernel(const _Float16* __restrict__ o,
                                                         const _Float16* __restrict__ z,
                                                         int rows, int d, float eps,
                                                         _Float16* __restrict__ y) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;  // (token, head) row
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const size_t base = static_cast<size_t>(row) * d;
  float ss = 0.0f;
  for (int c = lane; c < d; c += kWave) {
    const float v = static_cast<float>(o[base + c]);
    ss = fmaf(v, v, ss);
  }
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, kWave);
  const float inv = rsqrtf(ss / static_cast<float>(d) + eps);
  for (int c = lane; c < d; c += kWave) {
    const float zv = static_cast<float>(z[base + c]);
    y[base + c] = static_cast<_Float16>(static_cast<float>(o[base + c]) * inv * silu(zv));
  }
}

// ---------------------------------------------------------------------------
// workspace layout of one group call
// ---------------------------------------------------------------------------
struct Workspace {
  size_t xres, rs, p, q, k, v, z, la, be, o, y, ss, total;
};

Workspace plan(const LayerShape& L, int T) {
  Workspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes, kAlign);
    return at;
  };
  const size_t t = static_cast<size_t>(T);
  w.xres = take(t * L.hidden * 4);
  w.rs = take(t * 4);
  w.p = take(t * L.n_all() * 4);
  w.q = take(t * L.h_k * L.d * 2);
  w.k = take(t * L.h_k * L.d * 2);
  w.v = take(t * L.h_v * L.d * 2);
  w.z = take(t * L.h_v * L.d * 2);
  w.la = take(t * L.h_v * 4);
  w.be = take(t * L.h_v * 4);
  w.o = take(t * L.h_v * L.d * 2);
  w.y = take(t * L.h_v * L.d * 2);
  w.ss = take(t * 4);
  w.total = off;
  return w;
}

template <typename TA, int EPI, typename TX>
hipError_t gemm(const void* A, int lda, const _Float16* Bt, int ldb, int M, int N, int K,
                float* C, int ldc, const float* rs, const void* X, int ldx, hipStream_t s) {
  if (M == 0) return hipSuccess;
  dim3 grid(N / GBN, (M + GBM - 1) / GBM), block(256);
  hipLaunchKernelGGL((gemm_kernel<TA, EPI, TX>), grid, block, 0, s, A, lda, Bt, ldb, M, N, K, C,
                     ldc, rs, X, ldx);
  return hipGetLastError();
}

bool shape_ok(const sr_group_desc* d) {
  return d->hidden > 0 && d->hidden % 128 == 0 && d->h_k > 0 && d->h_v > 0 &&
         d->h_v % d->h_k == 0 && (d->d == 64 || d->d == 128) && d->conv_width >= 2 &&
         d->conv_width <= 8 && d->n_seqs >= 0 && d->total_tokens >= 0;
}

}  // namespace
}  // namespace sr

using sr::LayerShape;

extern "C" size_t sr_packed_layer_bytes(int32_t hidden, int32_t h_k, int32_t h_v, int32_t d,
                                        int32_t conv_width) {
  if (hidden <= 0 || h_k <= 0 || h_v <= 0 || d <= 0 || conv_width <= 0) return 0;
  LayerShape L{hidden, h_k, h_v, d, conv_width};
  return L.total();
}

extern "C" int sr_pack_gdn_layer(const void* w_in, const void* conv_w, const void* w_out,
                                 int32_t hidden, int32_t h_k, int32_t h_v, int32_t d,
                                 int32_t conv_width, void* packed, void* stream) {
  if (!w_in || !conv_w || !packed) return SR_EINVAL;
  if (hidden <= 0 || hidden % 128 != 0 || h_k <= 0 || h_v <= 0 || h_v % h_k != 0 ||
      (d != 64 && d != 128) || conv_width < 2 || conv_width > 8)
    return SR_ESHAPE;
  if ((reinterpret_cast<uintptr_t>(packed) & (sr::kAlign - 1)) != 0) return SR_EINVAL;
  LayerShape L{hidden, h_k, h_v, d, conv_width};
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(packed);
  _Float16* win = reinterpret_cast<_Float16*>(base);
  float* conv = reinterpret_cast<float*>(base + L.win_bytes());
  _Float16* wout = reinterpret_cast<_Float16*>(base + L.win_bytes() + L.conv_bytes());
  hipLaunchKernelGGL(sr::pack_win_kernel, dim3(2048), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w_in), L, win);
  hipLaunchKernelGGL(sr::pack_win_copy_kernel, dim3(4096), dim3(256), 0, s,
                     static_cast<const uint16_t*>(w_in), L, win);
  hipLaunchKernelGGL(sr::pack_conv_kernel, dim3(256), dim3(256), 0, s,
                     static_cast<const uint16_t*>(conv_w), L, conv);
  if (w_out)
    hipLaunchKernelGGL(sr::pack_wout_kernel, dim3(4096), dim3(256), 0, s,
                       static_cast<const uint16_t*>(w_out), L, wout);
  return hipGetLastError() == hipSuccess ? SR_OK : SR_ELAUNCH;
}

extern "C" size_t sr_replay_group_workspace_bytes(const sr_group_desc* d) {
  if (!d || !sr::shape_ok(d)) return 0;
  LayerShape L{d->hidden, d->h_k, d->h_v, d->d, d->conv_width};
  return sr::plan(L, d->total_tokens).total;
}

extern "C" int sr_replay_group(const sr_group_desc* d, const sr_gdn_layer_weights* weights,
                               const void* anchors, const int32_t* cu_seqlens, float* states,
                               float* conv_states, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!d || (d->n_layers > 0 && !d->layer_kind)) return SR_EINVAL;
  if (!sr::shape_ok(d) || d->n_layers < 0) return SR_ESHAPE;
  // the GDN layers must form one contiguous run; FA layers lead or trail
  int n_gdn = 0, first = -1, last = -1;
  for (int i = 0; i < d->n_layers; ++i) {
    const int k = d->layer_kind[i];
    if (k != SR_LAYER_GDN && k != SR_LAYER_FA) return SR_EINVAL;
    if (k == SR_LAYER_GDN) {
      if (last >= 0 && last != i - 1) return SR_ESHAPE;
      if (first < 0) first = i;
      last = i;
      ++n_gdn;
    }
  }
  if (n_gdn == 0 || d->n_seqs == 0) return SR_OK;
  if (!weights || !cu_seqlens || !states) return SR_EINVAL;
  for (int i = 0; i < n_gdn; ++i)
    if (!weights[i].packed) return SR_EINVAL;
  LayerShape L{d->hidden, d->h_k, d->h_v, d->d, d->conv_width};
  const int T = d->total_tokens;
  const sr::Workspace W = sr::plan(L, T);
  if (T > 0 && (!anchors || !workspace)) return SR_EINVAL;
  if (T > 0 && workspace_bytes < W.total) return SR_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (sr::kAlign - 1)) != 0) return SR_EINVAL;
  if ((reinterpret_cast<uintptr_t>(anchors) & 15u) != 0) return SR_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* xres = reinterpret_cast<float*>(ws + W.xres);
  float* rs = reinterpret_cast<float*>(ws + W.rs);
  float* P = reinterpret_cast<float*>(ws + W.p);
  _Float16* qb = reinterpret_cast<_Float16*>(ws + W.q);
  _Float16* kb = reinterpret_cast<_Float16*>(ws + W.k);
  _Float16* vb = reinterpret_cast<_Float16*>(ws + W.v);
  _Float16* zb = reinterpret_cast<_Float16*>(ws + W.z);
  float* la = reinterpret_cast<float*>(ws + W.la);
  float* be = reinterpret_cast<float*>(ws + W.be);
  _Float16* ob = reinterpret_cast<_Float16*>(ws + W.o);
  _Float16* yb = reinterpret_cast<_Float16*>(ws + W.y);
  int32_t* sst = reinterpret_cast<int32_t*>(ws + W.ss);
  const size_t state_stride = static_cast<size_t>(d->n_seqs) * d->h_v * d->d * d->d;
  const size_t conv_stride = static_cast<size_t>(d->n_seqs) * L.conv_dim() * (L.width - 1);

  if (T > 0) {
    hipLaunchKernelGGL(sr::seq_start_kernel, dim3((T + 255) / 256), dim3(256), 0, s, cu_seqlens,
                       d->n_seqs, T, sst);
    if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
  }
  for (int li = 0; li < n_gdn; ++li) {
    const bool is_last = li == n_gdn - 1;
    const char* pk = static_cast<const char*>(weights[li].packed);
    const _Float16* win = reinterpret_cast<const _Float16*>(pk);
    const float* convw = reinterpret_cast<const float*>(pk + L.win_bytes());
    const _Float16* wout = reinterpret_cast<const _Float16*>(pk + L.win_bytes() + L.conv_bytes());
    float* st = states + state_stride * li;
    if (T > 0) {
      // x of this layer: the anchors (bf16) for the first, the residual after
      const bool from_anchors = li == 0;
      if (from_anchors)
        hipLaunchKernelGGL(sr::rms_rows_kernel<sr::BF16>, dim3((T + 3) / 4), dim3(256), 0, s,
                           anchors, T, d->hidden, d->rms_eps, rs);
      else
        hipLaunchKernelGGL(sr::rms_rows_kernel<sr::F32>, dim3((T + 3) / 4), dim3(256), 0, s,
                           static_cast<const void*>(xres), T, d->hidden, d->rms_eps, rs);
      if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
      // the last layer needs k|v|a|b for its state, and q as well when its
      // conv window is returned (q follows the state prefix in the packing)
      const int N = !is_last ? L.n_all()
                  : conv_states ? static_cast<int>(sr::align_up(L.q_off() + d->h_k * d->d, 128))
                                : L.n_state_pad();
      hipError_t e =
          from_anchors
              ? sr::gemm<sr::BF16, sr::EPI_SCALE, sr::F32>(anchors, d->hidden, win, d->hidden, T, N,
                                                          d->hidden, P, L.n_all(), rs, nullptr, 0, s)
              : sr::gemm<sr::F32, sr::EPI_SCALE, sr::F32>(xres, d->hidden, win, d->hidden, T, N,
                                                         d->hidden, P, L.n_all(), rs, nullptr, 0, s);
      if (e != hipSuccess) return SR_ELAUNCH;
      hipLaunchKernelGGL(sr::frontend_kernel, dim3(T), dim3(256), 0, s, P, L.n_all(), L, convw, sst,
                         T, d->l2_eps, is_last, qb, kb, vb, zb, la, be);
      if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
      if (conv_states) {
        hipLaunchKernelGGL(sr::conv_state_kernel, dim3(64, d->n_seqs), dim3(256), 0, s, P, L.n_all(),
                           L, cu_seqlens, d->n_seqs, conv_states + conv_stride * li);
        if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
      }
    } else if (conv_states) {
      // no replayed tokens: the conv windows are empty (a fill kernel, not a
      // memset, so the call stays safe to capture in a graph)
      hipLaunchKernelGGL(sr::fill_kernel, dim3(256), dim3(256), 0, s,
                         conv_states + conv_stride * li, conv_stride, 0.0f);
      if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
    }
    sr::GdnArgs g{};
    g.n_seqs = d->n_seqs;
    g.total_tokens = T;
    g.h_k = d->h_k;
    g.h_v = d->h_v;
    g.d_k = d->d;
    g.d_v = d->d;
    g.dtype_qkv = SR_F16;
    g.dtype_o = SR_F16;
    g.erase = 1;
    g.alpha_is_log = 1;
    g.scale = 1.0f;
    g.q = is_last ? nullptr : qb;
    g.k = kb;
    g.v = vb;
    g.alpha = la;
    g.beta = be;
    g.cu = cu_seqlens;
    g.s0 = nullptr;
    g.s_out = st;
    g.o = is_last ? nullptr : ob;
    if (sr::launch_gdn_chunk(g, s) != hipSuccess) return SR_ELAUNCH;
    if (is_last || T == 0) continue;
    const int rows = T * d->h_v;
    hipLaunchKernelGGL(sr::gated_norm_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, ob, zb, rows,
                       d->d, d->rms_eps, yb);
    if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
    const int K2 = d->h_v * d->d;
    hipError_t e = li == 0 ? sr::gemm<sr::F16, sr::EPI_RESID, sr::BF16>(
                                 yb, K2, wout, K2, T, d->hidden, K2, xres, d->hidden, nullptr,
                                 anchors, d->hidden, s)
                           : sr::gemm<sr::F16, sr::EPI_RESID, sr::F32>(
                                 yb, K2, wout, K2, T, d->hidden, K2, xres, d->hidden, nullptr,
                                 xres, d->hidden, s);
    if (e != hipSuccess) return SR_ELAUNCH;
  }
  return SR_OK;
}
