// Replay of one group of linear-attention layers from its entry anchors
// ("SuffixReplay", Algorithm Design 1: one anchor per group, only the linear
// layers run, full-attention layers are skipped; "Tail-Replay", section 3:
// zero initial state per group, the group's final FFN omitted).
//
// Per GDN layer (pre-norm residual block without FFN):
//   xh   = fp16(x / sqrt(mean x^2 + eps))                  rms_norm_kernel
//   P    = xh W_in (fp16), packed columns k|v|a|b|pad|q|z  gemm_kernel (MFMA)
//   q,k  = L2norm(SiLU(conv(P_q,P_k))), v = SiLU(conv(P_v)),
//   log a = -softplus(P_a), b = sigmoid(P_b)               frontend_kernel
//   (for conv widths up to 4 with zero history the projection and the conv,
//   SiLU and L2 norms are one kernel, gemm_front_kernel, and P keeps only
//   z and a|b; gates_kernel forms the gates)
//   S, o = gated delta rule from S_0 = 0                   launch_gdn_chunk
//   y    = rms(o) o SiLU(P_z) per value head               gated_norm_kernel
//   x    = x + y W_out (fp32, in the projection's epilogue) gemm_kernel (MFMA)
// The last GDN layer of the group only needs its state: its projection
// covers the k|v|a|b prefix of the packed columns (plus q when the conv
// windows are returned) and no output is formed.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
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
__global__ void pack_win_kernel(LayerShape L, _Float16* __restrict__ wt) {
  const size_t total = static_cast<size_t>(L.n_all()) * L.hidden;
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<size_t>(gridDim.x) * blockDim.x)
    wt[e] = static_cast<_Float16>(0.0f);
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

// FFN weights: gate, up bf16 [hidden][F] -> W_gu^T fp16 [2F][hidden] with rows
// alternating in pairs (gate c, up c, gate c+1, up c+1, ...: the layout the
// EPI_SWIGLU epilogue reads); down bf16 [F][hidden] -> W_down^T fp16
// [hidden][F]
__global__ void pack_ffn_kernel(const uint16_t* __restrict__ wg, const uint16_t* __restrict__ wu,
                                const uint16_t* __restrict__ wd, int hidden, int F,
                                _Float16* __restrict__ gu, _Float16* __restrict__ dn) {
  const size_t total = static_cast<size_t>(hidden) * F;
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < total;
       e += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int k = static_cast<int>(e / F), c = static_cast<int>(e % F);  // w*[k][c]
    // gate c at row 4 (c/2) + 2 (c%2), up c right after it
    const size_t row_g = static_cast<size_t>(4 * (c / 2) + 2 * (c % 2));
    gu[row_g * hidden + k] = static_cast<_Float16>(bf16_to_f32(wg[e]));
    gu[(row_g + 1) * hidden + k] = static_cast<_Float16>(bf16_to_f32(wu[e]));
    // down: e indexes [F][hidden] as well (same count)
    const int f = static_cast<int>(e / hidden), n = static_cast<int>(e % hidden);
    dn[static_cast<size_t>(n) * F + f] = static_cast<_Float16>(bf16_to_f32(wd[e]));
  }
}

// ---------------------------------------------------------------------------
// pre-mixer RMSNorm (unit weight): xh_t = fp16(x_t / sqrt(mean_c x_t,c^2 + eps)),
// one wave per row, 8 consecutive elements per lane and step
// ---------------------------------------------------------------------------
template <typename TX>
__device__ __forceinline__ void load8f(const void* x, size_t idx, float (&v)[8]);
template <>
__device__ __forceinline__ void load8f<BF16>(const void* x, size_t idx, float (&v)[8]) {
  const u16x8 b = *reinterpret_cast<const u16x8*>(static_cast<const uint16_t*>(x) + idx);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = bf16_to_f32(b[e]);
}
template <>
__device__ __forceinline__ void load8f<F32>(const void* x, size_t idx, float (&v)[8]) {
  const f32x4 lo = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + idx);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + idx + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = lo[e];
    v[4 + e] = hi[e];
  }
}

// One row per wave: the RMSNorm of x (the anchors in bf16, or the fp32
// residual stream) in fp16, the A operand of the next projection.
template <typename TX>
__global__ __launch_bounds__(256) void rms_norm_kernel(const void* x, int rows, int cols,
                                                       float eps, _Float16* __restrict__ xh) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= rows) return;
  const size_t base = static_cast<size_t>(row) * cols;
  float s = 0.0f;
  for (int c = 8 * lane; c < cols; c += 8 * kWave) {
    float v[8];
    load8f<TX>(x, base + c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(v[e], v[e], s);
  }
  const float r = rsqrtf(wave_sum(s) / static_cast<float>(cols) + eps);
  for (int c = 8 * lane; c < cols; c += 8 * kWave) {
    float v[8];
    load8f<TX>(x, base + c, v);
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(v[e] * r);
    *reinterpret_cast<f16x8*>(xh + base + c) = h;
  }
}

// ---------------------------------------------------------------------------
// C[M][N] = A[M][K] . Bt[N][K]^T on the matrix cores: fp16 operands, fp32
// accumulation.
//   EPI_STORE16: C fp16 = acc
//   EPI_STORE32: C fp32 = acc
//   EPI_ADD_F32, EPI_ADD_BF16: C fp32 = X + acc (the residual add of a
//                block's output projection; X fp32, in place allowed, or
//                the bf16 anchors)
//   EPI_SWIGLU:  B's rows alternate gate and up columns in pairs, so the
//                4 consecutive results of a lane are (g_c, u_c, g_c+1,
//                u_c+1); C fp16 [M][N/2] = SiLU(g) * u (the FFN's gated
//                product, formed in the epilogue)
// Workgroup tile 256 x 256 x 64, 4 waves of 128 x 128 (16 accumulators of
// 32x32x16 MFMAs each, held in the accumulation registers); LDS is double
// buffered, the next k-tile is loaded into registers while the current one
// is multiplied, so each k-tile costs one barrier.  One workgroup per CU.
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so each XCD is
// given a contiguous range of a grouped order (8 M-tiles wide, walking N):
// the ~32 tiles an XCD runs at a time share 8 A and 4 B panels in its L2.
// Leftover tiles of a last, partly filled round (a launch of 260 tiles on
// 256 CUs would otherwise take two full tile times): up to 16 of them run
// as 32 x 32 blocks, one wave each (gemm_block_kernel); more, up to 64, in
// the narrow variant (NJ = 1): the tile split into four 256 x 64 strips, one
// per workgroup (4 waves of 128 x 32).  Every output element is accumulated
// by the same MFMA sequence over the same k order in all of them, so results
// do not depend on which kernel computed them.
// Requirements: K % 64 == 0, N % 4 == 0, lda/ldb/ldc multiples of 8; M and
// N are guarded.
// ---------------------------------------------------------------------------
constexpr int EPI_STORE16 = 0;
constexpr int EPI_STORE32 = 1;
constexpr int EPI_SWIGLU = 2;
// residual adds: C = X + A B^T in fp32, X fp32 (may be C itself: each element
// is read and written by the same thread) or bf16 (the anchors)
constexpr int EPI_ADD_F32 = 3;
constexpr int EPI_ADD_BF16 = 4;
constexpr int GBM = 256, GBN = 256, GBK = 64, GLD = GBK + 8;
constexpr int GGROUP = 8;  // M-tiles per group of the tile order
constexpr int kXcdG = 8;   // XCDs
constexpr int kStrips = 4; // 64-column strips per tile (narrow variant)

// Tile (tm, tn) at position q of the grouped order.
__device__ __forceinline__ void gemm_tile_at(int q, int n_m, int n_n, int& tm, int& tn) {
  const int group = q / (GGROUP * n_n), first = group * GGROUP;
  const int gsz = min(n_m - first, GGROUP);
  tm = first + (q % (GGROUP * n_n)) % gsz;
  tn = (q % (GGROUP * n_n)) / gsz;
}

// Main loop of one tile: rows m0 .. m0+255 of A (clamped into [0, M)),
// columns n0 .. n0+64NJ-1 of Bt (clamped below N), all of K.  sm: the
// kernel's LDS, [2][GBM*GLD + 64NJ*GLD] halves.  On return acc holds C^T
// fragments: lane l has row m0 + wm*128 + 32i + l%32 and, in register group
// g = r/4, columns n0 + wn*32NJ + 32j + 8g + 4(l/32) .. +3.
template <int NJ>
__device__ __forceinline__ void gemm_mainloop(const _Float16* __restrict__ A, int lda,
                                              const _Float16* __restrict__ Bt, int ldb, int M,
                                              int N, int K, int m0, int n0, _Float16* sm_,
                                              f32x16 (&acc)[4][NJ]) {
  constexpr int BN = 64 * NJ;                 // columns of the workgroup
  constexpr int SB = GBM * GLD + BN * GLD;    // halves per buffer
  constexpr int LOADS = GBM * GBK / 8 / 256;  // 16-byte A loads per thread
  constexpr int LOADB = BN * GBK / 8 / 256;   // 16-byte B loads per thread
  _Float16 (*sm)[SB] = reinterpret_cast<_Float16 (*)[SB]>(sm_);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = tid % kWave;
  const int wm = w / 2, wn = w % 2;

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // Thread tid moves the 16-byte pieces (row tid/8 + 32e, chunk tid%8) of
  // each operand tile.  Rows outside [0, M) (N) are clamped into range: they
  // are computed and never stored, and the loop stays branch-free.  Byte
  // offsets fit in 32 bits (the launcher splits larger problems), so a load
  // is one instruction: uniform base (k0) + per-thread offset.
  uint32_t aoff[LOADS], boff[LOADB];
#pragma unroll
  for (int e = 0; e < LOADS; ++e) {
    const int row = tid / (GBK / 8) + (256 / (GBK / 8)) * e, ch = tid % (GBK / 8);
    aoff[e] = static_cast<uint32_t>(
        (static_cast<size_t>(min(max(m0 + row, 0), M - 1)) * lda + 8 * ch) * 2);
  }
#pragma unroll
  for (int e = 0; e < LOADB; ++e) {
    const int row = tid / (GBK / 8) + (256 / (GBK / 8)) * e, ch = tid % (GBK / 8);
    boff[e] = static_cast<uint32_t>((static_cast<size_t>(min(n0 + row, N - 1)) * ldb + 8 * ch) * 2);
  }
  u32x4 ra[LOADS], rb[LOADB];
  auto gload_a = [&](int k0, int e) {
    ra[e] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(A + k0) + aoff[e]);
  };
  auto gload_b = [&](int k0, int e) {
    rb[e] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(Bt + k0) + boff[e]);
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int e = 0; e < LOADS; ++e) {
      const int row = tid / (GBK / 8) + (256 / (GBK / 8)) * e, ch = tid % (GBK / 8);
      *reinterpret_cast<u32x4*>(&sm[buf][row * GLD + 8 * ch]) = ra[e];
      if (e < LOADB) *reinterpret_cast<u32x4*>(&sm[buf][GBM * GLD + row * GLD + 8 * ch]) = rb[e];
    }
  };

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // lane l reads rows/columns l % 32 of each 32-wide fragment, k 8(l/32)..+7
  f16x8 av[2][4], bv[2][NJ];
  auto load_frag = [&](int buf, int ks, f16x8(&fa)[4], f16x8(&fb)[NJ]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      fa[i] = *reinterpret_cast<const f16x8*>(&sm[buf][(wm * 128 + 32 * i + l % 32) * GLD + 16 * ks + 8 * (l / 32)]);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      fb[j] = *reinterpret_cast<const f16x8*>(
          &sm[buf][GBM * GLD + (wn * 32 * NJ + 32 * j + l % 32) * GLD + 16 * ks + 8 * (l / 32)]);
  };
  // C^T tiles (B fragment as the first operand): a lane then holds 4
  // consecutive columns of one row, so the epilogue stores 4 values at once
  auto mma = [&](int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = mfma32x32x16(bv[h][j], av[h][i], acc[i][j]);
  };

  const int nk = K / GBK;
  if constexpr (NJ == 1) {
    // Strips do a quarter of a tile's MFMAs per k-tile, too few to cover a
    // k-tile of load latency: their loads run two k-tiles ahead, in two
    // register stages (k-tile kt+1 is stored to LDS at the end of k-tile kt,
    // k-tile kt+2 is issued at its start).  Same k order as the tiles.
    u32x4 ra2[LOADS], rb2[LOADB];
    auto issue = [&](u32x4(&xa)[LOADS], u32x4(&xb)[LOADB], int kt) {
      const int k0 = min(kt, nk - 1) * GBK;
#pragma unroll
      for (int e = 0; e < LOADS; ++e)
        xa[e] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(A + k0) + aoff[e]);
#pragma unroll
      for (int e = 0; e < LOADB; ++e)
        xb[e] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(Bt + k0) + boff[e]);
    };
    auto stash = [&](const u32x4(&xa)[LOADS], const u32x4(&xb)[LOADB], int buf) {
#pragma unroll
      for (int e = 0; e < LOADS; ++e) {
        const int row = tid / (GBK / 8) + (256 / (GBK / 8)) * e, ch = tid % (GBK / 8);
        *reinterpret_cast<u32x4*>(&sm[buf][row * GLD + 8 * ch]) = xa[e];
        if (e < LOADB) *reinterpret_cast<u32x4*>(&sm[buf][GBM * GLD + row * GLD + 8 * ch]) = xb[e];
      }
    };
    auto step = [&](int buf) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        load_frag(buf, ks, av[0], bv[0]);
        mma(0);
      }
    };
    issue(ra, rb, 0);
    stash(ra, rb, 0);
    issue(ra, rb, 1);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 2) {
      issue(ra2, rb2, kt + 2);
      step(0);
      stash(ra, rb, 1);  // k-tile kt + 1
      __syncthreads();
      if (kt + 1 >= nk) break;
      issue(ra, rb, kt + 3);
      step(1);
      stash(ra2, rb2, 0);  // k-tile kt + 2
      __syncthreads();
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < LOADS; ++e) gload_a(0, e);
#pragma unroll
  for (int e = 0; e < LOADB; ++e) gload_b(0, e);
  store_tile(0);
  __syncthreads();
  // Per k-tile: four k16 steps of 4 NJ MFMAs per wave.  Interleaved with
  // them (full tiles): the next step's fragment reads, the next k-tile's
  // global loads (A in step 0, B in step 1) and its LDS stores (step 3, into
  // the other buffer).  The last k-tile reloads itself, so the body has no
  // branches.
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const int kn = (kt + 1 < nk ? kt + 1 : kt) * GBK;
    load_frag(buf, 0, av[0], bv[0]);
    __builtin_amdgcn_sched_barrier(0);
    // step 0
    load_frag(buf, 1, av[1], bv[1]);
#pragma unroll
    for (int e = 0; e < LOADS; ++e) gload_a(kn, e);
    mma(0);
    if constexpr (NJ == 4) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // step 1
    load_frag(buf, 2, av[0], bv[0]);
#pragma unroll
    for (int e = 0; e < LOADB; ++e) gload_b(kn, e);
    mma(1);
    if constexpr (NJ == 4) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // step 2
    load_frag(buf, 3, av[1], bv[1]);
    mma(0);
    if constexpr (NJ == 4) {
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // step 3
    store_tile(buf ^ 1);
    mma(1);
    if constexpr (NJ == 4) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }
}

// Epilogue of four consecutive results C[m][n..n+3] (n % 4 == 0), shared by
// every GEMM kernel so that all of them apply the same arithmetic.
template <int EPI>
__device__ __forceinline__ void gemm_store4(void* C, int ldc, const void* X, int ldx, int m, int n,
                                            f32x4 v) {
  const size_t ci = static_cast<size_t>(m) * ldc + n;
  if (EPI == EPI_STORE16) {
    *reinterpret_cast<f16x4*>(static_cast<_Float16*>(C) + ci) = to_f16x4(v);
  } else if (EPI == EPI_SWIGLU) {
    const f16x2 h = {static_cast<_Float16>(silu(v[0]) * v[1]),
                     static_cast<_Float16>(silu(v[2]) * v[3])};
    *reinterpret_cast<f16x2*>(static_cast<_Float16*>(C) + static_cast<size_t>(m) * ldc + n / 2) = h;
  } else if (EPI == EPI_ADD_F32 || EPI == EPI_ADD_BF16) {
    const size_t xi = static_cast<size_t>(m) * ldx + n;
    f32x4 x;
    if (EPI == EPI_ADD_F32) {
      x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(X) + xi);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = load1<BF16>(X, xi + e);
    }
    *reinterpret_cast<f32x4*>(static_cast<float*>(C) + ci) = x + v;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(C) + ci) = v;
  }
}

// Tiles q_begin .. q_begin + q_count - 1 of the grouped order: one per
// workgroup (NJ = 4), or one 64-column strip per workgroup (NJ = 1).
template <int EPI, int NJ>
__global__ __launch_bounds__(256, 1) void gemm_kernel(const _Float16* __restrict__ A, int lda,
                                                      const _Float16* __restrict__ Bt, int ldb,
                                                      int M, int N, int K, void* C, int ldc,
                                                      const void* X, int ldx, int q_begin,
                                                      int q_count) {
  constexpr int BN = 64 * NJ;                 // columns of the workgroup
  __shared__ _Float16 sm[2 * (GBM * GLD + BN * GLD)];  // [buffer][A rows | B rows]
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = tid % kWave;
  const int wm = w / 2, wn = w % 2;
  int tm, tn, strip = 0;
  {
    const int n_m = (M + GBM - 1) / GBM, n_n = (N + GBN - 1) / GBN;
    int q;
    if (NJ == 4) {
      const int per_xcd = (q_count + kXcdG - 1) / kXcdG;
      q = (blockIdx.x % kXcdG) * per_xcd + blockIdx.x / kXcdG;
      if (q >= q_count) return;
    } else {
      q = blockIdx.x / kStrips;
      strip = blockIdx.x % kStrips;
      if (q >= q_count) return;
    }
    gemm_tile_at(q_begin + q, n_m, n_n, tm, tn);
  }
  const int n0 = tn * GBN + BN * strip;
  const int m0 = tm * GBM;
  if (n0 >= N) return;  // a strip past the last column
  f32x16 acc[4][NJ];
  gemm_mainloop<NJ>(A, lda, Bt, ldb, M, N, K, m0, n0, sm, acc);
  // epilogue: lane holds row m = l%32 of fragment i and, in register group
  // g = r/4, columns 8g + 4(l/32) .. +3 of fragment j
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 128 + 32 * i + l % 32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 32 * NJ + 32 * j + 8 * g + 4 * (l / 32);
        if (n >= N) continue;  // N % 4 == 0: a group of 4 is in or out as a whole
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        gemm_store4<EPI>(C, ldc, X, ldx, m, n, v);
      }
  }
}

// A few tiles left over after the full rounds, as 32 x 32 blocks of C, one
// wave each: tile q_begin + b/64 of the grouped order, block (b%64)/8 of its
// rows and b%8 of its columns.  A handful of leftover tiles then spreads
// over the CUs instead of holding a few of them for a whole tile time.  The
// operands come straight from global memory (16-byte pieces, PF k-steps in
// flight); each element is accumulated by the same MFMA, with the B fragment
// first, over the same k order as in gemm_kernel, in one accumulation chain,
// so results do not depend on which kernel computed them.
template <int EPI>
__global__ __launch_bounds__(64) void gemm_block_kernel(const _Float16* __restrict__ A, int lda,
                                                        const _Float16* __restrict__ Bt, int ldb,
                                                        int M, int N, int K, void* C, int ldc,
                                                        const void* X, int ldx, int q_begin) {
  const int l = threadIdx.x;
  const int b = blockIdx.x;
  int tm, tn;
  gemm_tile_at(q_begin + b / 64, (M + GBM - 1) / GBM, (N + GBN - 1) / GBN, tm, tn);
  const int m0 = tm * GBM + 32 * ((b % 64) / 8);
  const int n0 = tn * GBN + 32 * (b % 8);
  if (m0 >= M || n0 >= N) return;
  // lane l: row l%32 of the A and Bt blocks (clamped into range: computed,
  // never stored), k 8(l/32)..+7 of each k16 step; 32-bit byte offsets from
  // a uniform base, as in gemm_kernel
  const uint32_t ao = static_cast<uint32_t>(
      (static_cast<size_t>(min(m0 + l % 32, M - 1)) * lda + 8 * (l / 32)) * 2);
  const uint32_t bo = static_cast<uint32_t>(
      (static_cast<size_t>(min(n0 + l % 32, N - 1)) * ldb + 8 * (l / 32)) * 2);
  const int ns = K / 16;  // k16 steps
  // PF steps in flight (2 PF loads outstanding, within the wait counter's
  // range); the chunks of PF steps have no branch between the MFMAs, so
  // each MFMA waits for its own operands only
  constexpr int PF = 16;
  f16x8 ar[PF], br[PF];
  auto load = [&](int p, int step) {
    const int k0 = 16 * min(step, ns - 1);  // past the end: reload the last step (never used)
    ar[p] = *reinterpret_cast<const f16x8*>(reinterpret_cast<const char*>(A + k0) + ao);
    br[p] = *reinterpret_cast<const f16x8*>(reinterpret_cast<const char*>(Bt + k0) + bo);
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) load(p, p);
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  const int nfull = ns / PF * PF;
  for (int s0 = 0; s0 < nfull; s0 += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      acc = mfma32x32x16(br[p], ar[p], acc);
      load(p, s0 + p + PF);
      // keep each refill next to its MFMA (left to itself the scheduler
      // sinks all refills to the end of the chunk, and the chunk's last
      // MFMA then waits for every load in flight)
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the last ns - nfull steps (K % (16 PF) != 0) sit in slots 0, 1, ...
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < ns - nfull) acc = mfma32x32x16(br[p], ar[p], acc);
  // lane l: row m0 + l%32; register group g: columns n0 + 8g + 4(l/32) .. +3
  const int m = m0 + l % 32;
  if (m >= M) return;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int n = n0 + 8 * g + 4 * (l / 32);
    if (n >= N) continue;  // N % 4 == 0: a group of 4 is in or out as a whole
    const f32x4 v = {acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
    gemm_store4<EPI>(C, ldc, X, ldx, m, n, v);
  }
}

// ---------------------------------------------------------------------------
// front end: one workgroup per 64-token block and 512 channels of one kind
// (k, v or q heads; grid y): causal depthwise conv over the projection rows
// (zero history before each token's sequence start, or the carried-in
// window) + SiLU, per-head L2 norm of q and k; the last y index does the
// gates of the block.  A wave walks 16 tokens with all the rows its window
// needs loaded up front; a lane owns 8 adjacent channels (one 16-byte load
// or store per row), so a head's 128 (64) channels sit in 16 (8) adjacent
// lanes and its L2 sum is a DPP butterfly within them.  z is not copied:
// the gated RMSNorm reads it from P.
// ---------------------------------------------------------------------------
constexpr int FT = 64;    // tokens per workgroup
constexpr int FCH = 512;  // channels per workgroup (8 per lane)

// Sum over the `n` (8 or 16) adjacent lanes of a head, in every such lane.
template <int CTRL>
__device__ __forceinline__ float dpp_all(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int LANES>
__device__ __forceinline__ float head_sum(float x) {
  x += dpp_all<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_all<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_all<0x141>(x);  // row_half_mirror: the other quad of the 8
  if (LANES == 16) x += dpp_all<0x140>(x);  // row_mirror: the other 8 of the 16
  return x;
}

// n_blocks: the y extent before the gate blocks, blocks per kind in
// kb[0..2] (k, v, q); conv0 (may be null): per sequence the last width-1
// pre-conv rows before its first token ([n][conv_dim][width-1], original
// q|k|v channel order, oldest first), used for the taps that reach before
// the sequence start (continuation from a reconstructed state); null means
// zero history.  MAXW: conv widths up to MAXW (4 or 8).  HIST: conv0 may be
// non-null (the replay path, without it, keeps a small fully unrolled body).
template <int D, int MAXW, bool HIST>
__global__ __launch_bounds__(256) void frontend_kernel(
    const _Float16* __restrict__ P, int ldp, LayerShape L, const float* __restrict__ convw,
    const int32_t* __restrict__ seq_start, const int32_t* __restrict__ seq_id,
    const float* __restrict__ conv0, int T, float l2_eps, int kb_k, int kb_v, int kb_q,
    _Float16* __restrict__ qo, _Float16* __restrict__ ko, _Float16* __restrict__ vo,
    float* __restrict__ la, float* __restrict__ be) {
  constexpr int CL = 8;                // channels per lane
  constexpr int LPH = D / CL;          // lanes per head
  constexpr int HPB = FCH / D;         // heads per workgroup
  const int t0 = blockIdx.x * FT;
  const int by = blockIdx.y;
  const int nk = L.h_k, nv = L.h_v, W = L.width;
  if (by == kb_k + kb_v + kb_q) {  // gates
    for (int e = threadIdx.x; e < FT * nv; e += blockDim.x) {
      const int t = t0 + e / nv, h = e % nv;
      if (t >= T) break;
      const size_t pr = static_cast<size_t>(t) * ldp;
      la[static_cast<size_t>(t) * nv + h] = -softplus(static_cast<float>(P[pr + L.a_off() + h]));
      be[static_cast<size_t>(t) * nv + h] = sigmoid(static_cast<float>(P[pr + L.b_off() + h]));
    }
    return;
  }
  // kind 0: k, 1: v, 2: q; pbase / obase: packed / original column of the
  // kind's first channel
  int kind, hb0, nh, pbase, obase;
  _Float16* out;
  if (by < kb_k) {
    kind = 0; hb0 = by * HPB; nh = nk; pbase = 0; obase = nk * D; out = ko;
  } else if (by < kb_k + kb_v) {
    kind = 1; hb0 = (by - kb_k) * HPB; nh = nv; pbase = nk * D; obase = 2 * nk * D; out = vo;
  } else {
    kind = 2; hb0 = (by - kb_k - kb_v) * HPB; nh = nk; pbase = L.q_off(); obase = 0; out = qo;
  }
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int hidx = hb0 + lane / LPH;          // this lane's head
  const bool live = hidx < nh;
  const int cin = CL * (lane % LPH);          // first channel within the head
  const int pc = pbase + hidx * D + cin;      // packed column
  const int ch0 = conv_channel(L, pc);        // conv channels ch0 .. ch0+7
  const int oc = obase + hidx * D + cin;      // original q|k|v channel
  float wt[CL][MAXW];  // wt[e][k]: tap applied to row t-k
#pragma unroll
  for (int e = 0; e < CL; ++e)
#pragma unroll
    for (int k = 0; k < MAXW; ++k) wt[e][k] = live && k < W ? convw[(ch0 + e) * W + (W - 1 - k)] : 0.0f;
  // all input rows of this wave's 16 tokens are loaded up front (rows
  // tb-MAXW+1 .. tb+15; those before the window or outside [0, T) read 0)
  const int tb = t0 + 16 * wv;
  constexpr int NR = 16 + MAXW - 1;
  f16x8 u[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int row = tb - (MAXW - 1) + r;
    const bool ok = live && row >= 0 && row < T && r >= MAXW - W;
    u[r] = ok ? *reinterpret_cast<const f16x8*>(P + static_cast<size_t>(row) * ldp + pc) : f16x8{};
  }
  // sequence starts (and ids) of the wave's 16 tokens, one per lane
  // (broadcast below)
  const int sq = seq_start[min(tb + lane % 16, T - 1)];
  const int sid = HIST && conv0 ? seq_id[min(tb + lane % 16, T - 1)] : 0;
  const int W1 = W - 1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tb + i;
    const int back = t < T ? t - __builtin_amdgcn_readlane(sq, i) : -1;  // rows t-back .. t: t's sequence
    float y[CL];
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < CL; ++e) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < MAXW; ++k) {  // row t-k is u[MAXW-1+i-k]
        // taps before the sequence start see zero (or the carried window);
        // selected rather than branched on, so the body stays branch-free
        float x = k <= back ? static_cast<float>(u[MAXW - 1 + i - k][e]) : 0.0f;
        if (HIST && k > back && conv0 && k < W && back >= 0 && live) {
          // row t-k lies k-back rows before the sequence start: entry
          // W-1-(k-back) of the carried-in window
          const int n = __builtin_amdgcn_readlane(sid, i);
          x = conv0[(static_cast<size_t>(n) * L.conv_dim() + oc + e) * W1 + (W1 - (k - back))];
        }
        acc = fmaf(wt[e][k], x, acc);
      }
      y[e] = acc * __builtin_amdgcn_rcpf(1.0f + __expf(-acc));  // SiLU
      ss = fmaf(y[e], y[e], ss);
    }
    if (kind != 1) {
      const float inv = rsqrtf(head_sum<LPH>(ss) + l2_eps);
#pragma unroll
      for (int e = 0; e < CL; ++e) y[e] *= inv;
    }
    if (t < T && live) {
      f16x8 o;
#pragma unroll
      for (int e = 0; e < CL; ++e) o[e] = static_cast<_Float16>(y[e]);
      *reinterpret_cast<f16x8*>(out + (static_cast<size_t>(t) * nh + hidx) * D + cin) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Input projection fused with the front end (conv widths up to 4 with zero
// history): the same main loop as gemm_kernel, then the tile goes through
// LDS in fp16 (the values the separate front end would read from P) and the
// front end runs on it, so the conv channels of P never reach HBM; z is
// stored to P for the gated RMSNorm, a and b become the gates.  M tiles
// overlap by 3 rows: tile tm computes rows 253 tm - 3 .. 253 tm + 252 and
// emits the last 253, so every emitted row has its three conv predecessors
// in the tile.  Every value is computed exactly as gemm_kernel<EPI_STORE16>
// followed by frontend_kernel computes it (same fp16 rounding, tap order,
// SiLU and L2 sum).  A lane owns 8 adjacent columns of the tile and walks 32
// rows (16 in a half tile), four at a time.  The a|b columns go to P like z; gates_kernel
// forms the gates from them.
// ---------------------------------------------------------------------------
constexpr int FTM = GBM - 3;   // rows emitted per tile
constexpr int FTS = GBN + 8;   // row stride (halves) of the staged tile

// NJF = 4: whole 256-column tiles q_begin .. q_begin + q_count - 1 of the
// grouped order; NJF = 2: the same tiles as two 128-column halves each (one
// per workgroup; a half holds whole heads), for the tiles of a last, partly
// filled round when their halves fit in one round.  Each element is
// accumulated and finished exactly as in a whole tile.
template <int D, int NJF>
__global__ __launch_bounds__(256, 1) void gemm_front_kernel(
    const _Float16* __restrict__ A, int lda, const _Float16* __restrict__ Bt, int ldb, int M,
    int N, int K, LayerShape L, const float* __restrict__ convw,
    const int32_t* __restrict__ seq_start, float l2_eps, _Float16* __restrict__ P, int ldp,
    _Float16* __restrict__ qo, _Float16* __restrict__ ko, _Float16* __restrict__ vo, int q_begin,
    int q_count) {
  static_assert(NJF == 4 || NJF == 2, "whole tiles or halves");
  constexpr int BNF = 64 * NJF;     // columns of the workgroup
  constexpr int LPR = BNF / 8;      // lanes per tile row in the front end (8 columns each)
  constexpr int RPG = GBM * LPR / 256;  // rows walked by each lane group
  __shared__ _Float16 sm[2 * (GBM * GLD + GBN * GLD)];
  __shared__ int sst[GBM];
  static_assert(GBM * FTS <= 2 * (GBM * GLD + GBN * GLD), "staged tile must fit the LDS buffers");
  constexpr int LPH = D / 8;  // lanes per head
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l = tid % kWave;
  const int wm = w / 2, wn = w % 2;
  int tm, tn, half = 0;
  {
    const int n_m = (M + FTM - 1) / FTM, n_n = (N + GBN - 1) / GBN;
    int q;
    if (NJF == 4) {
      const int per_xcd = (q_count + kXcdG - 1) / kXcdG;
      q = (blockIdx.x % kXcdG) * per_xcd + blockIdx.x / kXcdG;
    } else {
      q = blockIdx.x / 2;
      half = blockIdx.x % 2;
    }
    if (q >= q_count) return;
    gemm_tile_at(q_begin + q, n_m, n_n, tm, tn);
  }
  const int n0 = tn * GBN + BNF * half;
  if (n0 >= N) return;  // a half past the last column
  const int m0 = tm * FTM - 3;
  f32x16 acc[4][NJF];
  gemm_mainloop<NJF>(A, lda, Bt, ldb, M, N, K, m0, n0, sm, acc);
  // (the main loop ends with a barrier: its LDS buffers are free)
  {
    const int t = m0 + tid;
    sst[tid] = t >= 0 && t < M ? seq_start[t] : 0;
  }
  _Float16* const T16 = sm;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJF; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = wm * 128 + 32 * i + l % 32;
        const int col = wn * 32 * NJF + 32 * j + 8 * g + 4 * (l / 32);
        const f32x4 v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
        *reinterpret_cast<f16x4*>(T16 + row * FTS + col) = to_f16x4(v);
      }
  __syncthreads();

  // this lane's 8 columns and what they are
  const int cb = l % LPR;
  const int col = n0 + 8 * cb;
  const int hk = L.h_k, hv = L.h_v;
  int kind = -1, hidx = 0, nh = 1, cin = 0;  // 0 k, 1 v, 2 q, 3 gates, 4 z
  _Float16* out = nullptr;
  if (col < N) {
    if (col < hk * D) {
      kind = 0; hidx = col / D; nh = hk; out = ko; cin = col % D;
    } else if (col < L.n_kv()) {
      kind = 1; hidx = (col - hk * D) / D; nh = hv; out = vo; cin = (col - hk * D) % D;
    } else if (col < L.n_state()) {
      kind = 3;
    } else if (col >= L.q_off() && col < L.q_off() + hk * D) {
      kind = 2; hidx = (col - L.q_off()) / D; nh = hk; out = qo; cin = (col - L.q_off()) % D;
    } else if (col >= L.z_off() && col < L.z_off() + hv * D) {
      kind = 4;
    }
  }
  const bool conv = kind >= 0 && kind <= 2;
  const int ch0 = conv ? conv_channel(L, col) : 0;
  const int W = L.width;
  float wt[8][4];  // wt[e][k]: tap applied to row t-k
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int k = 0; k < 4; ++k) wt[e][k] = conv && k < W ? convw[(ch0 + e) * W + (W - 1 - k)] : 0.0f;

  const int r0 = 3 + RPG * (w * (kWave / LPR) + l / LPR), r1 = min(r0 + RPG, GBM);
  // tiles without conv columns (z, pad) only copy z (and a|b) to P
  const bool any_conv = n0 < L.n_kv() || (n0 < L.q_off() + hk * D && n0 + BNF > L.q_off());
  if (!any_conv) {
    if (kind >= 3)
      for (int r = r0; r < r1 && m0 + r < M; ++r)
        *reinterpret_cast<f16x8*>(P + static_cast<size_t>(m0 + r) * ldp + col) =
            *reinterpret_cast<const f16x8*>(T16 + r * FTS + 8 * cb);
    return;
  }
  // rows r0 .. r1-1, four at a time (independent rows: their loads, conv,
  // SiLU and L2 sums overlap); u[j] / uf[j] hold row rb - 3 + j in fp16 (as
  // staged) and fp32 (each value converted once)
  f16x8 u[7];
  float uf[7][8];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    u[j] = *reinterpret_cast<const f16x8*>(T16 + (r0 - 3 + j) * FTS + 8 * cb);
#pragma unroll
    for (int e = 0; e < 8; ++e) uf[j][e] = static_cast<float>(u[j][e]);
  }
  for (int rb = r0; rb < r1; rb += 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u[3 + q] = *reinterpret_cast<const f16x8*>(T16 + min(rb + q, GBM - 1) * FTS + 8 * cb);
#pragma unroll
      for (int e = 0; e < 8; ++e) uf[3 + q][e] = static_cast<float>(u[3 + q][e]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = rb + q;
      const int t = m0 + r;
      const bool emit = r < r1 && t < M;  // uniform within each lane group of a row
      const int back = t - sst[min(r, GBM - 1)];  // rows t-back .. t belong to t's sequence
      float y[8];
      float ss = 0.0f;
      if (back >= 3) {  // every tap inside the sequence (the common case)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float a = 0.0f;
#pragma unroll
          for (int k = 0; k < 4; ++k) a = fmaf(wt[e][k], uf[3 + q - k][e], a);
          y[e] = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));  // SiLU
          ss = fmaf(y[e], y[e], ss);
        }
      } else {  // taps before the sequence start see zero
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float a = 0.0f;
#pragma unroll
          for (int k = 0; k < 4; ++k) a = fmaf(wt[e][k], k <= back ? uf[3 + q - k][e] : 0.0f, a);
          y[e] = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
          ss = fmaf(y[e], y[e], ss);
        }
      }
      const float inv = rsqrtf(head_sum<LPH>(ss) + l2_eps);  // every lane of the head takes part
      if (!emit) continue;
      if (conv) {
        f16x8 o;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = static_cast<_Float16>(kind != 1 ? y[e] * inv : y[e]);
        *reinterpret_cast<f16x8*>(out + (static_cast<size_t>(t) * nh + hidx) * D + cin) = o;
      } else if (kind >= 3) {
        // z, and the raw a|b columns (gates_kernel turns them into the gates:
        // the 8 lanes that hold them would otherwise hold up the tile)
        *reinterpret_cast<f16x8*>(P + static_cast<size_t>(t) * ldp + col) = u[3 + q];
      }
    }
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      u[j] = u[4 + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) uf[j][e] = uf[4 + j][e];
    }
  }
}

// Gates from the raw a|b projection columns: log a = -softplus(P_a),
// b = sigmoid(P_b), one thread per (token, value head).
__global__ __launch_bounds__(256) void gates_kernel(const _Float16* __restrict__ P, int ldp,
                                                    LayerShape L, int T, float* __restrict__ la,
                                                    float* __restrict__ be) {
  const size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  const int nv = L.h_v;
  if (e >= static_cast<size_t>(T) * nv) return;
  const size_t t = e / nv;
  const int h = static_cast<int>(e % nv);
  la[e] = -softplus(static_cast<float>(P[t * ldp + L.a_off() + h]));
  be[e] = sigmoid(static_cast<float>(P[t * ldp + L.b_off() + h]));
}

// conv state: last W-1 pre-conv rows of q|k|v per sequence (original
// channel order), oldest first, zero where the sequence is shorter
// (rows before the sequence start come from the carried-in window conv0,
// or are zero without one)
__global__ void conv_state_kernel(const _Float16* __restrict__ P, int ldp, LayerShape L,
                                  const int32_t* __restrict__ cu, int n_seqs,
                                  const float* __restrict__ conv0, float* __restrict__ out) {
  const int n = blockIdx.y;
  const int W1 = L.width - 1;
  const int cd = L.conv_dim();
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < cd * W1; e += gridDim.x * blockDim.x) {
    const int c = e / W1, j = e % W1;
    const int start = cu[n], end = cu[n + 1];
    const int pos = end - W1 + j;
    float v = 0.0f;
    if (pos >= start)
      v = static_cast<float>(P[static_cast<size_t>(pos) * ldp + L.packed_col(c)]);
    else if (conv0)
      v = conv0[(static_cast<size_t>(n) * cd + c) * W1 + (W1 - (start - pos))];
    out[(static_cast<size_t>(n) * cd + c) * W1 + j] = v;
  }
}

__global__ void copy_kernel(const float* __restrict__ src, float* __restrict__ dst, size_t n) {
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<size_t>(gridDim.x) * blockDim.x)
    dst[e] = src[e];
}

__global__ void fill_kernel(float* __restrict__ p, size_t n, float v) {
  for (size_t e = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; e < n;
       e += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[e] = v;
}

// seq_start[t] = cu[n] and seq_id[t] = n for the sequence n holding token t
__global__ void seq_start_kernel(const int32_t* __restrict__ cu, int n_seqs, int T,
                                 int32_t* __restrict__ out, int32_t* __restrict__ ids) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  out[t] = cu[lo];
  ids[t] = lo;
}

// out = x + dlt (the group's output hidden state: the last layer's residual
// stream plus its output projection), fp32

// y = o / sqrt(mean(o^2) + eps) * SiLU(z), per (token, value head), fp16 out;
// z is read from the projection rows (columns z_off + head * D).  A wave
// handles 4 rows, a lane D/64 adjacent elements of each; all loads of the 4
// rows are issued before any arithmetic.
template <int D>
__global__ __launch_bounds__(256) void gated_norm_kernel(const _Float16* __restrict__ o,
                                                         const _Float16* __restrict__ P, int ldp,
                                                         int z_off, int h_v, int rows, float eps,
                                                         _Float16* __restrict__ y) {
  constexpr int CPL = D / kWave, RPW = 4;
  typedef _Float16 h2 __attribute__((ext_vector_type(CPL)));
  const int lane = threadIdx.x % kWave;
  const int row0 = (blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave) * RPW;
  h2 ov[RPW], zv[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = min(row0 + r, rows - 1);
    ov[r] = *reinterpret_cast<const h2*>(o + static_cast<size_t>(row) * D + CPL * lane);
    zv[r] = *reinterpret_cast<const h2*>(P + static_cast<size_t>(row / h_v) * ldp + z_off +
                                         (row % h_v) * D + CPL * lane);
  }
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < CPL; ++e) ss = fmaf(static_cast<float>(ov[r][e]), static_cast<float>(ov[r][e]), ss);
    const float inv = rsqrtf(wave_sum(ss) / static_cast<float>(D) + eps);
    h2 out;
#pragma unroll
    for (int e = 0; e < CPL; ++e)
      out[e] = static_cast<_Float16>(static_cast<float>(ov[r][e]) * inv * silu(static_cast<float>(zv[r][e])));
    if (row0 + r < rows) *reinterpret_cast<h2*>(y + static_cast<size_t>(row0 + r) * D + CPL * lane) = out;
  }
}

// ---------------------------------------------------------------------------
// workspace layout of one group call
// ---------------------------------------------------------------------------
struct Workspace {
  size_t xres, xh, p, q, k, v, la, be, o, y, ss, sid, total;
};

// (the FFN's gated product [T][F] fp16 reuses the projection rows, dead by
// the time the FFN runs)
Workspace plan(const LayerShape& L, int T, int ffn_dim) {
  Workspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes, kAlign);
    return at;
  };
  const size_t t = static_cast<size_t>(T);
  w.xres = take(t * L.hidden * 4);
  w.xh = take(t * L.hidden * 2);
  w.p = take(t * static_cast<size_t>(std::max(L.n_all(), ffn_dim)) * 2);
  w.q = take(t * L.h_k * L.d * 2);
  w.k = take(t * L.h_k * L.d * 2);
  w.v = take(t * L.h_v * L.d * 2);
  w.la = take(t * L.h_v * 4);
  w.be = take(t * L.h_v * 4);
  w.o = take(t * L.h_v * L.d * 2);
  w.y = take(t * L.h_v * L.d * 2);
  w.ss = take(t * 4);
  w.sid = take(t * 4);
  w.total = off;
  return w;
}

template <int EPI>
hipError_t gemm(const _Float16* A, int lda, const _Float16* Bt, int ldb, int M, int N, int K,
                void* C, int ldc, hipStream_t s, const void* X = nullptr, int ldx = 0) {
  if (M == 0 || N == 0) return hipSuccess;
  // the kernel addresses A and Bt with 32-bit byte offsets: split M so that
  // every launch stays below 2^31 bytes of A
  const size_t row_bytes = static_cast<size_t>(lda) * 2;
  const int mc = static_cast<int>(std::max<size_t>(GBM, ((size_t{1} << 31) / row_bytes) / GBM * GBM));
  for (int m_at = 0; m_at < M; m_at += mc) {
    const int mm = std::min(mc, M - m_at);
    const int tiles = ((N + GBN - 1) / GBN) * ((mm + GBM - 1) / GBM);
    // Full rounds of whole tiles on the CUs; the tiles of a last, partly
    // filled round go out as 32 x 32 blocks (up to 16 tiles: one wave per
    // block, at most 4 blocks per CU) or as 64-column strips (up to 64
    // tiles: their strips fit in one round).  A strip does a quarter of a
    // tile's MFMAs but still streams the whole A panel and takes about half
    // a tile's time.  The 260 tiles of the 6552 x 2560 x 4096 output
    // projection: 205 us as two rounds, 124 + 61 us with the last 4 tiles as
    // 16 strips on 16 CUs, ~144 + 22 us with them as 160 blocks.
    int full = tiles, narrow = 0, blocks = 0;
    const int rest = tiles % kGfx950Cus;
    if (rest != 0 && 64 * rest <= 4 * kGfx950Cus) {
      full = tiles - rest;
      blocks = rest;
    } else if (rest != 0 && kStrips * rest <= kGfx950Cus) {
      full = tiles - rest;
      narrow = rest;
    }
    constexpr bool c32 = EPI == EPI_STORE32 || EPI == EPI_ADD_F32 || EPI == EPI_ADD_BF16;
    void* Cm = c32 ? static_cast<void*>(static_cast<float*>(C) + static_cast<size_t>(m_at) * ldc)
                   : static_cast<void*>(static_cast<_Float16*>(C) + static_cast<size_t>(m_at) * ldc);
    const void* Xm =
        EPI == EPI_ADD_F32    ? static_cast<const void*>(static_cast<const float*>(X) + static_cast<size_t>(m_at) * ldx)
        : EPI == EPI_ADD_BF16 ? static_cast<const void*>(static_cast<const uint16_t*>(X) + static_cast<size_t>(m_at) * ldx)
                              : nullptr;
    const _Float16* Am = A + static_cast<size_t>(m_at) * lda;
    if (full > 0) {
      dim3 grid((full + kXcdG - 1) / kXcdG * kXcdG), block(256);
      hipLaunchKernelGGL((gemm_kernel<EPI, 4>), grid, block, 0, s, Am, lda, Bt, ldb, mm, N, K, Cm,
                         ldc, Xm, ldx, 0, full);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (blocks > 0) {
      dim3 grid(blocks * 64), block(64);
      hipLaunchKernelGGL((gemm_block_kernel<EPI>), grid, block, 0, s, Am, lda, Bt, ldb, mm, N, K, Cm,
                         ldc, Xm, ldx, full);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (narrow > 0) {
      dim3 grid(narrow * kStrips), block(256);
      hipLaunchKernelGGL((gemm_kernel<EPI, 1>), grid, block, 0, s, Am, lda, Bt, ldb, mm, N, K, Cm,
                         ldc, Xm, ldx, full, narrow);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

bool shape_ok(const sr_group_desc* d) {
  return d->hidden > 0 && d->hidden % 128 == 0 && d->h_k > 0 && d->h_v > 0 &&
         d->h_v % d->h_k == 0 && (d->d == 64 || d->d == 128) && d->conv_width >= 2 &&
         d->conv_width <= 8 && d->n_seqs >= 0 && d->total_tokens >= 0 && d->ffn_dim >= 0 &&
         d->ffn_dim % 64 == 0;
}

}  // namespace
}  // namespace sr

using sr::LayerShape;

extern "C" size_t sr_packed_ffn_bytes(int32_t hidden, int32_t ffn_dim) {
  if (hidden <= 0 || ffn_dim <= 0) return 0;
  return sr::align_up(static_cast<size_t>(3) * ffn_dim * hidden * 2, sr::kAlign);
}

extern "C" int sr_pack_ffn(const void* w_gate, const void* w_up, const void* w_down,
                           int32_t hidden, int32_t ffn_dim, void* packed, void* stream) {
  if (!w_gate || !w_up || !w_down || !packed) return SR_EINVAL;
  if (hidden <= 0 || hidden % 128 != 0 || ffn_dim <= 0 || ffn_dim % 64 != 0) return SR_ESHAPE;
  if ((reinterpret_cast<uintptr_t>(packed) & (sr::kAlign - 1)) != 0) return SR_EINVAL;
  _Float16* gu = static_cast<_Float16*>(packed);
  _Float16* dn = gu + static_cast<size_t>(2 * ffn_dim) * hidden;
  hipLaunchKernelGGL(sr::pack_ffn_kernel, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint16_t*>(w_gate), static_cast<const uint16_t*>(w_up),
                     static_cast<const uint16_t*>(w_down), hidden, ffn_dim, gu, dn);
  return hipGetLastError() == hipSuccess ? SR_OK : SR_ELAUNCH;
}

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
  hipLaunchKernelGGL(sr::pack_win_kernel, dim3(2048), dim3(256), 0, s, L, win);
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
  return sr::plan(L, d->total_tokens, d->ffn_dim).total;
}

namespace sr {
namespace {

// The whole group replay on a given workspace (shared by the entry points).
// states0 / conv0 (may be null): per-layer states and conv windows to start
// from (continuation); hidden_out (may be null): the group's output hidden
// states, which makes the last layer run its full mixer as well.
int replay_group_run(const sr_group_desc* d, const sr_gdn_layer_weights* weights,
                     const void* anchors, const int32_t* cu_seqlens, const float* states0,
                     const float* conv0, float* states, float* conv_states, float* hidden_out,
                     void* workspace, size_t workspace_bytes, void* stream) {
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
  const sr::Workspace W = sr::plan(L, T, d->ffn_dim);
  if (T > 0 && (!anchors || !workspace)) return SR_EINVAL;
  if (T > 0 && workspace_bytes < W.total) return SR_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & (sr::kAlign - 1)) != 0) return SR_EINVAL;
  if ((reinterpret_cast<uintptr_t>(anchors) & 15u) != 0) return SR_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (sr::debug_checks_enabled()) {
    const int c = sr::check_cu_seqlens(cu_seqlens, d->n_seqs, T, s);
    if (c != SR_OK) return c;
  }
  char* ws = static_cast<char*>(workspace);
  float* xres = reinterpret_cast<float*>(ws + W.xres);
  _Float16* xh = reinterpret_cast<_Float16*>(ws + W.xh);
  _Float16* P = reinterpret_cast<_Float16*>(ws + W.p);
  _Float16* qb = reinterpret_cast<_Float16*>(ws + W.q);
  _Float16* kb = reinterpret_cast<_Float16*>(ws + W.k);
  _Float16* vb = reinterpret_cast<_Float16*>(ws + W.v);
  float* la = reinterpret_cast<float*>(ws + W.la);
  float* be = reinterpret_cast<float*>(ws + W.be);
  _Float16* ob = reinterpret_cast<_Float16*>(ws + W.o);
  _Float16* yb = reinterpret_cast<_Float16*>(ws + W.y);
  int32_t* sst = reinterpret_cast<int32_t*>(ws + W.ss);
  int32_t* sid = reinterpret_cast<int32_t*>(ws + W.sid);
  const size_t state_stride = static_cast<size_t>(d->n_seqs) * d->h_v * d->d * d->d;
  const size_t conv_stride = static_cast<size_t>(d->n_seqs) * L.conv_dim() * (L.width - 1);

  if (T > 0) {
    hipLaunchKernelGGL(sr::seq_start_kernel, dim3((T + 255) / 256), dim3(256), 0, s, cu_seqlens,
                       d->n_seqs, T, sst, sid);
    if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
  }
  // The residual stream x starts as the anchors (bf16); each block's output
  // projection adds its output to it in its epilogue, writing the fp32 sum
  // to xres (in place after the first), or to the group's output buffer for
  // the group's last block.
  bool x_is_anchors = true;
  auto norm = [&]() -> bool {
    const dim3 rgrid((T + 3) / 4);
    if (x_is_anchors)
      hipLaunchKernelGGL((sr::rms_norm_kernel<sr::BF16>), rgrid, dim3(256), 0, s, anchors, T,
                         d->hidden, d->rms_eps, xh);
    else
      hipLaunchKernelGGL((sr::rms_norm_kernel<sr::F32>), rgrid, dim3(256), 0, s,
                         static_cast<const void*>(xres), T, d->hidden, d->rms_eps, xh);
    return hipGetLastError() == hipSuccess;
  };
  // x <- x + A B^T: into xres, or into the output buffer when `out` is set
  auto add_block = [&](const _Float16* A, int lda, const _Float16* Bt, int K, float* out) -> bool {
    float* C = out ? out : xres;
    const hipError_t e =
        x_is_anchors
            ? sr::gemm<sr::EPI_ADD_BF16>(A, lda, Bt, K, T, d->hidden, K, C, d->hidden, s, anchors,
                                         d->hidden)
            : sr::gemm<sr::EPI_ADD_F32>(A, lda, Bt, K, T, d->hidden, K, C, d->hidden, s, xres,
                                        d->hidden);
    x_is_anchors = false;
    return e == hipSuccess;
  };
  for (int li = 0; li < n_gdn; ++li) {
    const bool is_last = li == n_gdn - 1;
    // the mixer's outputs are formed for every layer but the last, and for
    // the last too when the group's output is asked for
    const bool full = !is_last || hidden_out != nullptr;
    const float* lconv0 = conv0 ? conv0 + conv_stride * li : nullptr;
    const char* pk = static_cast<const char*>(weights[li].packed);
    const _Float16* win = reinterpret_cast<const _Float16*>(pk);
    const float* convw = reinterpret_cast<const float*>(pk + L.win_bytes());
    const _Float16* wout = reinterpret_cast<const _Float16*>(pk + L.win_bytes() + L.conv_bytes());
    float* st = states + state_stride * li;
    if (T > 0) {
      // x of this layer: the anchors for the first, after that the residual
      // stream; xh = RMSNorm(x) in fp16, the A operand of the projection
      if (!norm()) return SR_ELAUNCH;
      // the last layer needs k|v|a|b for its state, and q as well when its
      // conv window is returned (q follows the state prefix in the packing)
      const int N = full ? L.n_all()
                  : conv_states ? static_cast<int>(sr::align_up(L.q_off() + d->h_k * d->d, 128))
                                : L.n_state_pad();
      // Projection and front end in one kernel unless the conv needs a
      // carried window (extension), a width above 4, or P's conv columns
      // (the conv windows are returned), or A is too large for 32-bit offsets
      const bool fuse = L.width <= 4 && !lconv0 && !conv_states &&
                        static_cast<size_t>(T) * d->hidden * 2 < (size_t{1} << 31);
      if (fuse) {
        // A projection of at most 128 tiles (a small batch) runs as 256
        // 128-column halves, so it spreads over twice as many CUs.  Larger
        // ones stay whole tiles in one launch: a second launch for the
        // halves of a partly filled last round waits for the first to drain,
        // which measured slower than the one launch, whose last tiles start
        // as CUs free up (96,829 tokens: 24.1 against 23.9 ms per group).
        const int n_m = (T + sr::FTM - 1) / sr::FTM, n_n = (N + sr::GBN - 1) / sr::GBN;
        const int tiles = n_m * n_n;
        const int halves = 2 * tiles <= kGfx950Cus ? tiles : 0;
        const int whole = tiles - halves;
        auto front = [&](auto kern, int nblk, int q0, int nq) {
          if (nq == 0) return hipSuccess;
          hipLaunchKernelGGL(kern, dim3(nblk), dim3(256), 0, s, xh, d->hidden, win, d->hidden, T, N,
                             d->hidden, L, convw, sst, d->l2_eps, P, L.n_all(), qb, kb, vb, q0, nq);
          return hipGetLastError();
        };
        const int gw = (whole + sr::kXcdG - 1) / sr::kXcdG * sr::kXcdG;
        hipError_t e1, e2;
        if (d->d == 128) {
          e1 = front(sr::gemm_front_kernel<128, 4>, gw, 0, whole);
          e2 = front(sr::gemm_front_kernel<128, 2>, 2 * halves, whole, halves);
        } else {
          e1 = front(sr::gemm_front_kernel<64, 4>, gw, 0, whole);
          e2 = front(sr::gemm_front_kernel<64, 2>, 2 * halves, whole, halves);
        }
        if (e1 != hipSuccess || e2 != hipSuccess) return SR_ELAUNCH;
        const size_t ng = static_cast<size_t>(T) * d->h_v;
        hipLaunchKernelGGL(sr::gates_kernel, dim3(static_cast<unsigned>((ng + 255) / 256)), dim3(256),
                           0, s, P, L.n_all(), L, T, la, be);
        if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
      } else {
      if (sr::gemm<sr::EPI_STORE16>(xh, d->hidden, win, d->hidden, T, N, d->hidden, P, L.n_all(),
                                    s) != hipSuccess)
        return SR_ELAUNCH;
      // conv heads: k, v (and q unless this is the last layer), then gates
      const int hpb = sr::FCH / d->d;  // heads per front-end workgroup
      const int kb_k = (d->h_k + hpb - 1) / hpb, kb_v = (d->h_v + hpb - 1) / hpb;
      const int kb_q = full ? kb_k : 0;
      const dim3 fgrid((T + sr::FT - 1) / sr::FT, kb_k + kb_v + kb_q + 1);
      auto fe = lconv0 ? (d->d == 128 ? (L.width <= 4 ? sr::frontend_kernel<128, 4, true>
                                                      : sr::frontend_kernel<128, 8, true>)
                                      : (L.width <= 4 ? sr::frontend_kernel<64, 4, true>
                                                      : sr::frontend_kernel<64, 8, true>))
                       : (d->d == 128 ? (L.width <= 4 ? sr::frontend_kernel<128, 4, false>
                                                      : sr::frontend_kernel<128, 8, false>)
                                      : (L.width <= 4 ? sr::frontend_kernel<64, 4, false>
                                                      : sr::frontend_kernel<64, 8, false>));
      hipLaunchKernelGGL(fe, fgrid, dim3(256), 0, s, P, L.n_all(), L, convw, sst, sid, lconv0, T,
                         d->l2_eps, kb_k, kb_v, kb_q, qb, kb, vb, la, be);
      if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
      }
      if (conv_states) {
        hipLaunchKernelGGL(sr::conv_state_kernel, dim3(64, d->n_seqs), dim3(256), 0, s, P, L.n_all(),
                           L, cu_seqlens, d->n_seqs, lconv0, conv_states + conv_stride * li);
        if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
      }
    } else if (conv_states) {
      // no tokens: the conv windows are the carried-in ones, or empty (kernels,
      // not memset/memcpy nodes, so the call stays safe to capture in a graph)
      if (lconv0)
        hipLaunchKernelGGL(sr::copy_kernel, dim3(256), dim3(256), 0, s, lconv0,
                           conv_states + conv_stride * li, conv_stride);
      else
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
    g.q = full ? qb : nullptr;
    g.k = kb;
    g.v = vb;
    g.alpha = la;
    g.beta = be;
    g.cu = cu_seqlens;
    g.s0 = states0 ? states0 + state_stride * li : nullptr;
    g.s_out = st;
    g.o = full ? ob : nullptr;
    if (sr::launch_gdn_chunk(g, s) != hipSuccess) return SR_ELAUNCH;
    // layer-wise handoff: this layer's state and conv window are final now
    if (d->layer_events && d->layer_events[li]) {
      if (hipEventRecord(static_cast<hipEvent_t>(d->layer_events[li]), s) != hipSuccess)
        return SR_ELAUNCH;
    }
    if (!full || T == 0) continue;
    const int rows = T * d->h_v;
    const dim3 ngrid((rows + 15) / 16);
    if (d->d == 128)
      hipLaunchKernelGGL(sr::gated_norm_kernel<128>, ngrid, dim3(256), 0, s, ob, P, L.n_all(),
                         L.z_off(), d->h_v, rows, d->rms_eps, yb);
    else
      hipLaunchKernelGGL(sr::gated_norm_kernel<64>, ngrid, dim3(256), 0, s, ob, P, L.n_all(),
                         L.z_off(), d->h_v, rows, d->rms_eps, yb);
    if (hipGetLastError() != hipSuccess) return SR_ELAUNCH;
    const int K2 = d->h_v * d->d;
    // FFN block after the mixer (not after the last layer of a replay: its
    // output is never used there): x <- x + W_down (SiLU(xh W_g) * (xh W_u))
    const bool has_ffn = d->ffn_dim > 0 && weights[li].ffn;
    // x <- x + y W_out; the group's last block writes the sum, the group's
    // output, to hidden_out
    if (!add_block(yb, K2, wout, K2, is_last && !has_ffn ? hidden_out : nullptr))
      return SR_ELAUNCH;
    if (has_ffn) {
      const int F = d->ffn_dim;
      const _Float16* wgu = static_cast<const _Float16*>(weights[li].ffn);
      const _Float16* wdn = wgu + static_cast<size_t>(2 * F) * d->hidden;
      _Float16* hb = P;  // [T][F] fp16, the projection rows are dead here
      if (!norm()) return SR_ELAUNCH;
      if (sr::gemm<sr::EPI_SWIGLU>(xh, d->hidden, wgu, d->hidden, T, 2 * F, d->hidden, hb, F, s) !=
          hipSuccess)
        return SR_ELAUNCH;
      if (!add_block(hb, F, wdn, F, is_last ? hidden_out : nullptr)) return SR_ELAUNCH;
    }
  }
  return SR_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the workspace is a file-scope device array of
// kScratchBytes per GPU (allocated with the code object, held until the
// process ends).  Host code never passes the array's name to a kernel: the
// device address comes from hipGetSymbolAddress, looked up once per device
// with that device current.  Every call on a GPU reuses that GPU's array, so
// calls that overlap on one GPU race; nothing in it has to start at zero
// (each kernel of the group writes every workspace element it later reads).
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t{256} << 20;
constexpr int kMaxDevices = 64;

}  // namespace

__device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

int scratch_ptr(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SR_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return SR_EDEVICE;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SR_EDEVICE;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return SR_OK;
}

}  // namespace
}  // namespace sr

extern "C" int sr_replay_group(const sr_group_desc* d, const sr_gdn_layer_weights* weights,
                               const void* anchors, const int32_t* cu_seqlens, float* states,
                               float* conv_states, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return sr::replay_group_run(d, weights, anchors, cu_seqlens, nullptr, nullptr, states,
                              conv_states, nullptr, workspace, workspace_bytes, stream);
}

extern "C" int sr_extend_group(const sr_group_desc* d, const sr_gdn_layer_weights* weights,
                               const void* tokens, const int32_t* cu_seqlens,
                               const float* initial_states, const float* initial_conv_states,
                               float* states, float* conv_states, float* hidden_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return sr::replay_group_run(d, weights, tokens, cu_seqlens, initial_states,
                              initial_conv_states, states, conv_states, hidden_out, workspace,
                              workspace_bytes, stream);
}

extern "C" size_t sr_replay_group_noalloc_max_bytes(void) { return sr::kScratchBytes; }

extern "C" int sr_replay_group_noalloc(const sr_group_desc* d,
                                       const sr_gdn_layer_weights* weights,
                                       const void* anchors, const int32_t* cu_seqlens,
                                       float* states, float* conv_states, void* stream) {
  if (!d || (d->n_layers > 0 && !d->layer_kind)) return SR_EINVAL;
  if (!sr::shape_ok(d) || d->n_layers < 0) return SR_ESHAPE;
  // the size check comes first: a call that does not fit touches nothing
  if (sr_replay_group_workspace_bytes(d) > sr::kScratchBytes) return SR_EWORKSPACE;
  void* ws = nullptr;
  const int st = sr::scratch_ptr(&ws);
  if (st != SR_OK) return st;
  return sr::replay_group_run(d, weights, anchors, cu_seqlens, nullptr, nullptr, states,
                              conv_states, nullptr, ws, sr::kScratchBytes, stream);
}
