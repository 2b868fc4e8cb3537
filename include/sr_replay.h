/*
 * sr_replay.h -- C ABI of the suffix-replay state reconstruction library
 * (MI355X / gfx950).
 *
 * On a prefix-cache hit, a hybrid model's linear-attention (Gated DeltaNet)
 * states are rebuilt by replaying only the last k cached anchor hidden states
 * of the matched prefix through each group of linear layers, from a zero
 * state, skipping full-attention layers ("SuffixReplay", Theoretical
 * Foundation Eq. 1-2 and 4, Algorithm Design 1-3; "Tail-Replay", section 3).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers unless marked "host".  The
 *    caller owns every buffer (inputs, outputs and workspaces); the library
 *    allocates no device memory and keeps no pointer after a call returns.
 *  - Calls enqueue work on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream) and return without synchronising.
 *  - Arguments are checked on the host first.  On any failure nothing is
 *    enqueued and a nonzero SR_E* code is returned (sr_status_str() names
 *    it).  A failed kernel launch returns SR_ELAUNCH.
 *  - Preconditions that live in device memory are documented, and checked
 *    only on request: cu_seqlens non-decreasing with cu[0] = 0 and
 *    cu[N] = total_tokens; alpha in (0, 1] (log alpha in [-inf, 0]; values
 *    below -64 are clamped); beta in [0, 2]; replay lengths 0 <= k_i <= m_i
 *    and page ids in range.  sr_check_replay_inputs / sr_check_gather_inputs
 *    run a validation kernel over them and return SR_EDATA on a violation
 *    (they synchronise the stream).  With the environment variable SR_DEBUG
 *    set to 1, every entry point runs the matching check first and returns
 *    its status before anything else is enqueued.
 *  - Packed varlen tensors are token-major: row t of a [T][...] tensor holds
 *    token t of the concatenation of all sequences, as cu_seqlens splits it.
 *  - Results are deterministic (no atomics in reductions): repeated calls on
 *    the same inputs give bit-identical outputs.
 *  - Calls that share a stream are ordered; the library holds no global
 *    mutable state and is reentrant.
 */
#ifndef SR_REPLAY_H_
#define SR_REPLAY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define SR_OK 0
#define SR_EINVAL 1     /* null required pointer, bad enum or flag          */
#define SR_ESHAPE 2     /* unsupported or inconsistent sizes                */
#define SR_EDTYPE 3     /* unsupported dtype combination                    */
#define SR_EWORKSPACE 4 /* workspace missing or too small                   */
#define SR_ELAUNCH 5    /* a kernel launch failed (HIP error)               */
#define SR_EDEVICE 6    /* no usable gfx950 device                          */
#define SR_EDATA 7      /* device-side inputs break a documented precondition
                           (only reported by the validation checks)         */

/* element types */
#define SR_BF16 0
#define SR_F16 1
#define SR_F32 2

/* layer kinds of a replay group */
#define SR_LAYER_GDN 0
#define SR_LAYER_FA 1

/* Library version string, static storage. */
const char* sr_version(void);

/* Human-readable name of a status code, static storage. */
const char* sr_status_str(int status);

/* --------------------------------------------------------------------------
 * Gated-delta-rule replay of one linear-attention layer.
 *
 * Defines ("SuffixReplay", Eq. 4, with A_t = decay + rank-one erase;
 * "Tail-Replay", section 2: gate alpha in (0,1] and a rank-1 correction),
 * per sequence n and value head h, with S a d_v x d_k matrix:
 *
 *   erase = 1:  S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *   erase = 0:  S_t = alpha_t S_{t-1} + beta_t v_t k_t^T   (scalar decay only)
 *   S_0 = initial_state (or 0, the replay case),  o_t = scale * S_t q_t.
 *
 * Value head h reads query/key head h / (h_v / h_k) (contiguous groups).
 *
 * Layouts (row-major, packed varlen, T = total_tokens):
 *   q, k          [T][h_k][d_k]   dtype_qkv
 *   v             [T][h_v][d_v]   dtype_qkv
 *   alpha         [T][h_v] fp32   alpha, or log(alpha) if alpha_is_log
 *   beta          [T][h_v] fp32   or NULL for beta = 1
 *   cu_seqlens    [n_seqs+1] int32 (device)
 *   initial_state [n_seqs][h_v][d_k][d_v] fp32 or NULL (= 0)
 *   final_state   [n_seqs][h_v][d_k][d_v] fp32, required; the TRANSPOSE of
 *                 S (row j = key index, column i = value index)
 *   o             [T][h_v][d_v]   dtype_o, or NULL (state only; q may then
 *                 be NULL)
 *
 * Supported: dtype_qkv SR_BF16 / SR_F16 with d_k = d_v in {64, 128} run the
 * chunked kernel (chunks of 64 tokens, fp16 matrix-core operands, fp32
 * accumulation and fp32 state); dtype_qkv SR_F32 (any d_k, d_v in {32, 64,
 * 128}) runs a token-serial fp32 kernel.  bf16 inputs are converted to fp16
 * on load, which is exact for |x| in [2^-14, 65504]; larger magnitudes are
 * outside the contract.  dtype_o: SR_BF16, SR_F16 or SR_F32.
 * n_seqs = 0 or total_tokens = 0 is allowed; an empty sequence returns its
 * initial state.
 *
 * State magnitude: the chunked kernel keeps each wave's part of the state as
 * 2^E times a register copy (E >= 0 chosen per chunk), so the fp16 operand
 * copies of the state stay in range for states of any fp32 magnitude.
 *
 * Workspace: sr_gdn_workspace_bytes() bytes (currently 0 for every
 * supported shape; workspace may then be NULL).  Status: SR_EINVAL for a
 * null required pointer, a bad flag or a misaligned q/k/v/o (16-byte rows,
 * 8-byte outputs); SR_ESHAPE for unsupported sizes; SR_EDTYPE;
 * SR_EWORKSPACE; SR_ELAUNCH.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_seqs;       /* N >= 0                                          */
  int32_t total_tokens; /* T >= 0, must equal cu_seqlens[N] (not checked)  */
  int32_t h_k, h_v;     /* h_v % h_k == 0                                  */
  int32_t d_k, d_v;
  int32_t dtype_qkv;    /* SR_BF16 | SR_F16 | SR_F32                       */
  int32_t dtype_o;      /* SR_BF16 | SR_F16 | SR_F32                       */
  int32_t erase;        /* 1 = gated delta rule, 0 = decay-only            */
  int32_t alpha_is_log; /* 1: alpha holds log(alpha) <= 0                  */
  float scale;          /* output scale, usually 1                         */
} sr_gdn_desc;

typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const float* alpha;
  const float* beta;
  const int32_t* cu_seqlens;
  const float* initial_state;
  float* final_state;
  void* o;
} sr_gdn_io;

/* Workspace bytes sr_gdn_replay_state needs for this descriptor (0 when it
 * needs none; (size_t)-1 for a descriptor it rejects). */
size_t sr_gdn_workspace_bytes(const sr_gdn_desc* desc);

int sr_gdn_replay_state(const sr_gdn_desc* desc, const sr_gdn_io* io,
                        void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Single-token decode step from a reconstructed state ("Tail-Replay",
 * section 3: the unmatched tokens continue from the reconstructed linear-
 * attention states; "SuffixReplay", Eq. 4 for one more token).  The same
 * recurrence and layouts as sr_gdn_replay_state with exactly one token per
 * sequence: desc->total_tokens must equal desc->n_seqs, row n of q, k, v,
 * alpha, beta and o belongs to sequence n, io->cu_seqlens is ignored.
 * io->initial_state is the state before the token (NULL = 0) and
 * io->final_state the state after it; they may be the same buffer (an
 * in-place update).  d_k = d_v in {64, 128}; any input dtype; fp32 state
 * arithmetic.  State buffers 8-byte aligned.  Memory-bound: each (sequence,
 * head) state is read once and written once.
 * ------------------------------------------------------------------------ */
int sr_gdn_decode_step(const sr_gdn_desc* desc, const sr_gdn_io* io, void* stream);

/* Validation of the device-side preconditions of one sr_gdn_replay_state
 * call (cu_seqlens, alpha, beta as described above).  Runs a kernel on
 * `stream`, waits for it and returns SR_OK, SR_EDATA, or the host-side
 * argument status of sr_gdn_replay_state. */
int sr_check_replay_inputs(const sr_gdn_desc* desc, const sr_gdn_io* io, void* stream);

/* --------------------------------------------------------------------------
 * Anchor gather and varlen packing ("SuffixReplay", Algorithm Design 2:
 * anchors on 64-token pages; System Design: hits packed into one variable-
 * length batch with device-side boundaries).
 *
 * For request i with matched length m_i and replay length k_i (0 <= k_i <=
 * m_i), packed rows cu[i] .. cu[i]+k_i-1 receive prefix positions
 * m_i-k_i .. m_i-1; position p lives in page page_table[i*pt_stride + p/64]
 * at row p % 64.  cu is the exclusive prefix sum of k (cu[0] = 0).
 *
 *   pool        [n_pages][64][hidden] (elem_bytes per element; copied
 *               bitwise, any 2- or 4-byte type)
 *   page_table  [n_req][pt_stride] int32 (device)
 *   matched_len [n_req] int32 (device), suffix_len [n_req] int32 (device)
 *   packed      [total_tokens][hidden], total_tokens = sum k_i (host value,
 *               must match the device data; rows beyond sum k_i are left
 *               untouched)
 *   cu_seqlens_out [n_req+1] int32
 * hidden * elem_bytes must be a multiple of 16.  The host-side total keeps
 * the launch free of a device-to-host read.  The pool may also live in
 * pinned host memory (hipHostMalloc; "SuffixReplay", System Design, Anchor
 * Sidecar: anchors can stay in host DRAM while KV pages stay in HBM): the
 * kernel then reads the anchor rows over the host link and writes the packed
 * rows to device memory, so a gather issued on its own stream overlaps work
 * on others.  A host pool that is not pinned and device-mapped is rejected
 * with SR_EINVAL.  Out-of-range page ids and
 * page-table columns are clamped (the launch stays in bounds; the copied
 * rows are then meaningless): sr_check_gather_inputs reports them.
 * ------------------------------------------------------------------------ */
int sr_gather_suffix(const void* pool, int32_t hidden, int32_t elem_bytes,
                     int64_t n_pages, const int32_t* page_table,
                     int32_t pt_stride, const int32_t* matched_len,
                     const int32_t* suffix_len, int32_t n_req,
                     int32_t total_tokens, void* packed,
                     int32_t* cu_seqlens_out, void* stream);

/* --------------------------------------------------------------------------
 * Gather with token-wise sparse anchors ("SuffixReplay", Algorithm Design 2,
 * Figure 3: anchors kept at a subset of positions aligned with the 64-token
 * pages, e.g. density 1/16; sampled densely next to the page boundary; and
 * Algorithm Design 3: the replay length counts anchors).
 *
 * Every 64-token page p of a prefix owns one anchor block of A rows (the
 * block sits in the same page slot, so the KV page table indexes it); row j
 * of the block holds the anchor at position 64 p + page_offsets[j].  A = 64
 * with offsets 0..63 is the dense case (sr_gather_suffix); density 1/16
 * sampled next to the boundary is A = 4 with offsets 60, 61, 62, 63.
 *
 * Request i's anchors are the positions 64 p + page_offsets[j] < m_i in
 * increasing order, n_i = A floor(m_i / 64) + #{j : page_offsets[j] <
 * m_i mod 64} of them; the packed rows cu[i] .. cu[i]+k_i-1 receive its
 * last k_i anchors (0 <= k_i <= n_i), and positions_out (may be NULL) the
 * prefix position of each packed row.
 *
 *   pool          [n_blocks][A][hidden], elem_bytes per element (bitwise)
 *   page_offsets  HOST [A], strictly increasing, in [0, 64); 1 <= A <= 64
 *   page_table, matched_len (tokens), suffix_len (anchors), cu_seqlens_out
 *                 as for sr_gather_suffix
 *   positions_out [total_tokens] int32 or NULL
 * ------------------------------------------------------------------------ */
int sr_gather_anchors(const void* pool, int32_t hidden, int32_t elem_bytes,
                      int64_t n_blocks, int32_t anchors_per_page,
                      const int32_t* page_offsets, const int32_t* page_table,
                      int32_t pt_stride, const int32_t* matched_len,
                      const int32_t* suffix_len, int32_t n_req,
                      int32_t total_tokens, void* packed,
                      int32_t* cu_seqlens_out, int32_t* positions_out,
                      void* stream);

/* Validation of a gather's device-side preconditions: m_i >= 0,
 * 0 <= k_i <= n_i (the anchors of request i; n_i = m_i for dense
 * anchors), every page-table column a replay reads below pt_stride and its
 * page id in [0, n_blocks), and sum k_i = total_tokens.  anchors_per_page /
 * page_offsets as for sr_gather_anchors (64 and NULL for dense anchors).
 * Runs a kernel, waits for it, returns SR_OK, SR_EDATA or a host-side
 * argument status. */
int sr_check_gather_inputs(int64_t n_blocks, int32_t anchors_per_page,
                           const int32_t* page_offsets, const int32_t* page_table,
                           int32_t pt_stride, const int32_t* matched_len,
                           const int32_t* suffix_len, int32_t n_req,
                           int32_t total_tokens, void* stream);

/* Replay budget ("SuffixReplay", Algorithm Design 3: the replay length, in
 * anchors, is min(0.05 n, k_max); "Tail-Replay", section 3: a fixed share
 * of the matched prefix).  k[i] = min(ceil(ratio * n_anchors[i]), k_max),
 * n_anchors[i] the anchors of request i's matched prefix; k_max <= 0 means
 * no cap.  Host function (host arrays); returns sum k[i], or -1 for bad
 * arguments (ratio outside (0, 1], a negative count, n_req < 0). */
int64_t sr_replay_budget(const int32_t* n_anchors, int32_t n_req, double ratio,
                         int32_t k_max, int32_t* k);

/* --------------------------------------------------------------------------
 * Replay of one group of linear-attention layers from its entry anchors
 * ("SuffixReplay", Algorithm Design 1: one group-entry anchor per group,
 * only linear layers run, full-attention layers are skipped; "Tail-Replay",
 * section 3: zero initial state per group, the group's final FFN omitted).
 *
 * Each GDN layer l (pre-norm residual block, no FFN; the layer internals are
 * not written out on the pages, the readings taken are):
 *   xh = x / sqrt(mean(x^2) + rms_eps)                   (unit weight)
 *   [q|k|v|z|a|b] = xh W_in      W_in [hidden][n_in], n_in = 2 h_k d +
 *                                 2 h_v d + 2 h_v
 *   c = SiLU(causal depthwise conv of q|k|v, width conv_width, zero history)
 *   q, k = per-head c / sqrt(|c|^2 + l2_eps);  v = c
 *   log alpha = -softplus(a), beta = sigmoid(b)
 *   S_l, o = gdn replay (erase mode, S_0 = 0)
 *   layers before the last:  x <- x + (rms(o) * SiLU(z)) W_out   (gated
 *   RMSNorm per value head, unit weight, rms_eps), W_out [h_v d][hidden]
 *   the last GDN layer only produces its state.
 *
 * Weights come pre-packed (sr_pack_gdn_layer): the matrix-core kernels read
 * them k-contiguous in fp16, and a layer's weights are static, so the
 * re-layout is done once when the weights are loaded rather than on every
 * replay.  The raw bf16 {w_in, conv_w, w_out} triple is what
 * sr_pack_gdn_layer takes.
 *
 *   anchors     [T][hidden] bf16
 *   cu_seqlens  [n_seqs+1] int32 (device)
 *   states      [n_gdn][n_seqs][h_v][d][d] fp32 (transposed S per head, as
 *               final_state above)
 *   conv_states [n_gdn][n_seqs][conv_dim][conv_width-1] fp32 or NULL: the
 *               last conv_width-1 pre-conv rows of q|k|v per sequence,
 *               oldest first, zero where a sequence is shorter (asking for
 *               them makes the last layer project its q columns too)
 *   workspace   >= sr_replay_group_workspace_bytes(desc) bytes, 256-aligned
 *
 * Supported: h_v % h_k == 0, d in {64, 128}, conv_width in 2..8,
 * hidden % 128 == 0.  FA layers may lead or trail the GDN layers but not sit
 * between them (one anchor tensor feeds one contiguous run of GDN layers).
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t n_layers;
  const int32_t* layer_kind; /* host [n_layers]: SR_LAYER_GDN | SR_LAYER_FA */
  int32_t hidden, h_k, h_v, d, conv_width;
  float rms_eps, l2_eps;
  int32_t n_seqs, total_tokens, max_seqlen;
  /* Layer-wise handoff ("SuffixReplay", System Design, Pipelined Replay
   * Path: a consumer waits only for the layer whose state it reads): host
   * array [n_gdn] of hipEvent_t (as void*), or NULL.  Entry l, if not NULL,
   * is recorded on the stream right after GDN layer l's state (and conv
   * window) is written, so another stream can hipStreamWaitEvent on it
   * instead of on the whole group. */
  void* const* layer_events;
  /* FFN width of the layers' feed-forward blocks (0: no FFN), a multiple of
   * 64.  A layer whose weights carry an FFN (sr_gdn_layer_weights.ffn) runs
   * x <- x + W_down (SiLU(RMSNorm(x) W_gate) * (RMSNorm(x) W_up)) after its
   * mixer ("Tail-Replay", section 3: replay omits the group's final FFN:
   * the last layer's FFN runs only when the group's output hidden states
   * are asked for, sr_extend_group). */
  int32_t ffn_dim;
} sr_group_desc;

/* Packed weights of one GDN layer, produced by sr_pack_gdn_layer into a
 * caller-owned buffer of sr_packed_layer_bytes() bytes. */
typedef struct {
  const void* packed; /* device, 256-aligned: sr_pack_gdn_layer output        */
  const void* ffn;    /* device, 256-aligned: sr_pack_ffn output, or NULL (no
                         FFN block after this layer)                          */
} sr_gdn_layer_weights;

/* Size in bytes of one packed layer for these shapes. */
size_t sr_packed_layer_bytes(int32_t hidden, int32_t h_k, int32_t h_v,
                             int32_t d, int32_t conv_width);

/* Pack one layer: w_in bf16 [hidden][n_in], conv_w bf16 [conv_dim][width],
 * w_out bf16 [h_v d][hidden] (may be NULL when the layer is only ever used
 * as the last of a group) -> packed (device, sr_packed_layer_bytes bytes).
 * Converts to the fp16 k-contiguous layouts the kernels read; exact for
 * weights with |w| >= 2^-14 or w = 0, and within 2^-25 absolute below. */
int sr_pack_gdn_layer(const void* w_in, const void* conv_w, const void* w_out,
                      int32_t hidden, int32_t h_k, int32_t h_v, int32_t d,
                      int32_t conv_width, void* packed, void* stream);

/* FFN block of one layer: w_gate, w_up bf16 [hidden][ffn_dim], w_down bf16
 * [ffn_dim][hidden] -> packed (device, sr_packed_ffn_bytes bytes): fp16,
 * k-contiguous, gate and up columns interleaved in pairs so the gate|up
 * product and SiLU(g) * u come out of one matrix-core pass.  hidden % 128
 * == 0, ffn_dim % 64 == 0. */
size_t sr_packed_ffn_bytes(int32_t hidden, int32_t ffn_dim);
int sr_pack_ffn(const void* w_gate, const void* w_up, const void* w_down, int32_t hidden,
                int32_t ffn_dim, void* packed, void* stream);

size_t sr_replay_group_workspace_bytes(const sr_group_desc* desc);

int sr_replay_group(const sr_group_desc* desc,
                    const sr_gdn_layer_weights* weights /* host [n_gdn] */,
                    const void* anchors, const int32_t* cu_seqlens,
                    float* states, float* conv_states, void* workspace,
                    size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Continuation of a group from reconstructed states ("Tail-Replay",
 * section 3: the unmatched tokens continue from the reconstructed linear-
 * attention states; "SuffixReplay", System Design: replay and extend hand
 * over at group boundaries).  The new tokens of each sequence run through
 * the group's GDN layers as in sr_replay_group, but every layer starts from
 * its given state and short-conv window instead of zero:
 *   tokens               [T][hidden] bf16, the group input of the new tokens
 *   initial_states       [n_gdn][n_seqs][h_v][d][d] fp32 or NULL (= 0), the
 *                        layout sr_replay_group writes
 *   initial_conv_states  [n_gdn][n_seqs][conv_dim][conv_width-1] fp32 or
 *                        NULL (= zero history), the layout it writes
 *   states, conv_states  outputs as for sr_replay_group (conv_states may be
 *                        NULL); they must not alias the initial ones
 *   hidden_out           [T][hidden] fp32 or NULL: the group's output hidden
 *                        states (the last layer's residual plus its mixer
 *                        output; asking for it makes the last layer compute
 *                        its full mixer)
 * Workspace, errors and supported shapes as for sr_replay_group.  Replaying
 * a prefix and extending it by the rest equals replaying the whole sequence
 * up to rounding (chunk boundaries differ).
 * ------------------------------------------------------------------------ */
int sr_extend_group(const sr_group_desc* desc,
                    const sr_gdn_layer_weights* weights /* host [n_gdn] */,
                    const void* tokens, const int32_t* cu_seqlens,
                    const float* initial_states, const float* initial_conv_states,
                    float* states, float* conv_states, float* hidden_out,
                    void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Allocation-free group replay, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same computation, arguments, layouts and results as
 * sr_replay_group (bit-identical), but the workspace is a static device
 * array of sr_replay_group_noalloc_max_bytes() bytes (256 MiB) that the
 * library holds on every GPU it runs on until the process ends; the call
 * allocates and frees nothing.  A group whose workspace
 * (sr_replay_group_workspace_bytes) exceeds that size is rejected with
 * SR_EWORKSPACE before anything is enqueued (at hidden 2560 with 16 key /
 * 32 value heads of 128, about 3200 packed tokens fit).  All calls on one
 * GPU share the array: calls that overlap in time on one GPU (several host
 * threads, or several streams) race and give wrong results; serialise them.
 * SR_EDEVICE if the array's device address cannot be obtained.
 * ------------------------------------------------------------------------ */
size_t sr_replay_group_noalloc_max_bytes(void);

int sr_replay_group_noalloc(const sr_group_desc* desc,
                            const sr_gdn_layer_weights* weights /* host [n_gdn] */,
                            const void* anchors, const int32_t* cu_seqlens,
                            float* states, float* conv_states, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SR_REPLAY_H_ */
