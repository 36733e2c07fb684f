/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse Mixture-of-Experts layer library.
 *
 * The layer: a router scores every token against 256 experts, keeps the 8
 * best plus one shared expert that every token uses ("Lily: Perplexity's
 * Custom Inference Engine for Apple Silicon", section "The architecture that
 * forces the issue: MoE plus Gated DeltaNet"); routing histograms and block
 * maps stay on the GPU with no host round trip, and 4-bit expert weights are
 * rebuilt tile by tile inside the grouped GEMM, never written back expanded
 * ("Inside Lily: How Perplexity's Rust and Metal Engine Accelerates Qwen
 * Inference on Apple Silicon", section "Performance Gains and Workload
 * Patterns"); prefill runs as matrix-unit GEMMs and batch-1 decode as
 * bandwidth-bound GEMV on the vector ALUs (Lily page, section "Why Apple
 * Silicon isn't just a smaller datacenter GPU").
 *
 * Conventions for every entry point:
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates no device memory and keeps no device state between calls; the
 *     caller provides scratch memory as `workspace` where a call needs it.
 *     The one exception is moe_forward_noalloc(), whose scratch is a device
 *     array of the library itself (see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls enqueue their kernels on it and return without synchronising the
 *     host; results are ready when the stream reaches that point.
 *   - Arguments and shapes are validated on the host before anything is
 *     launched; a failed check returns its status and launches nothing.  A
 *     launch failure returns MOE_ERR_HIP (see moe_last_hip_error()).
 *   - Row-major layouts; bf16 and fp16 values are passed as uint16_t bit patterns.
 *   - Calls that share a workspace on one stream are ordered; calls that
 *     overlap on different streams must use different workspaces.
 *   - Every workspace (moe_forward's and moe_group's) starts with a 256-byte
 *     header whose first int32 is a device error word: kernels OR the
 *     MOE_DEVERR_* bits into it when they meet a condition that the host could
 *     not check before launch.  Read and clear it with moe_workspace_errors().
 *
 * Supported shapes: hidden % 64 == 0, inter % 64 == 0, shared_inter % 64 == 0,
 * group_size == 64, n_experts % 16 == 0 and 16 <= n_experts <= 256,
 * 1 <= top_k <= 16 (top_k <= n_experts), 1 <= T <= 65536.  These cover the
 * model (256 experts, top-8, groups of 64) with room on every side; wider
 * expert counts, k up to 32 and other group sizes are MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent arguments */
  MOE_ERR_UNSUPPORTED = -2, /* shape outside the supported set above */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  MOE_ERR_HIP = -4          /* a HIP launch failed */
} moe_status;

/* Bits of the device error word at the start of a workspace. */
enum {
  MOE_DEVERR_HANDOVER_TIMEOUT = 1, /* a wait of the fused 1-4-token layer gave up: that call's outputs are invalid */
  MOE_DEVERR_EXPERT_ID = 2         /* moe_group met an expert id outside [0, E): those slots were skipped, so
                                      counts, perm and the block map do not cover T*k slots */
};

/* Layer dimensions.  The workload model uses {2048, 512, 256, 8, 64, 512}. */
typedef struct moe_dims {
  int32_t hidden;       /* H: token width */
  int32_t inter;        /* I: intermediate width of a routed expert */
  int32_t n_experts;    /* E: routed experts */
  int32_t top_k;        /* k: experts kept per token */
  int32_t group_size;   /* G: int4 quantisation group along the input dim (64) */
  int32_t shared_inter; /* Is: intermediate width of the shared expert */
} moe_dims;

/* Affine int4 weights of n_exp experts (one matrix each), canonical layout:
 *   codes  uint8 [n_exp][N][K/2]: element (n, k) in byte k/2, low nibble = even k
 *   scales fp16  [n_exp][N][K/G], biases fp16 [n_exp][N][K/G]
 * Weight value w = bf16_rne( fp32(code) * fp32(scale) + fp32(bias) ).
 * gate_up matrices: N = 2*I (rows 0..I-1 gate, I..2I-1 up), K = H.
 * down matrices:    N = H, K = I.
 * `packed` is the same weights in the matrix-core layout written by
 * moe_prepack_q4() (NULL if not prepared): the grouped GEMMs read only it, the
 * fused path for 1-4 tokens reads only the canonical arrays. */
typedef struct moe_q4 {
  const uint8_t* codes;
  const uint16_t* scales;
  const uint16_t* biases;
  const uint8_t* packed;
} moe_q4;

/* Which matrix of a layer a moe_q4 holds (sets N, K and the column order). */
typedef enum moe_matrix {
  MOE_MAT_GATE_UP = 0,    /* routed experts: N = 2I, K = H */
  MOE_MAT_DOWN = 1,       /* routed experts: N = H,  K = I */
  MOE_MAT_SH_GATE_UP = 2, /* shared expert:  N = 2Is, K = H */
  MOE_MAT_SH_DOWN = 3     /* shared expert:  N = H,  K = Is */
} moe_matrix;

/* Bytes of the matrix-core layout of n_exp experts of one matrix kind
 * (0 for invalid arguments).  The layout: per expert, per slice of 256 product
 * columns, per 64-wide K block, one 9216-byte block holding the 256 columns'
 * 32 code bytes (in the order the GEMM's LDS stage uses) and then their
 * (fp16 scale, fp16 bias) pairs; gate/up slices interleave 32 gate and the
 * matching 32 up columns.  Columns past N are zero.  Same byte count as the
 * canonical arrays when N is a multiple of 256 (gate/up: I of 128). */
size_t moe_packed_q4_bytes(const moe_dims* d, int32_t matrix, int32_t n_exp);

/* Rewrite canonical weights w->codes/scales/biases of n_exp experts into the
 * matrix-core layout at `packed` (packed_bytes >= moe_packed_q4_bytes()).
 * A one-time weight preparation, like loading the checkpoint; values are
 * copied bit for bit, only their order changes. */
moe_status moe_prepack_q4(const moe_dims* d, int32_t matrix, const moe_q4* w, int32_t n_exp, uint8_t* packed,
                          size_t packed_bytes, void* stream);

/* All weights of one layer. */
typedef struct moe_layer {
  moe_q4 gate_up;              /* routed experts, [E][2I][H] */
  moe_q4 down;                 /* routed experts, [E][H][I] */
  moe_q4 sh_gate_up;           /* shared expert, [1][2Is][H] */
  moe_q4 sh_down;              /* shared expert, [1][H][Is] */
  const float* router_w;       /* [E][H] fp32; read by the fused path (1-4 tokens) */
  const float* router_bias;    /* [E] fp32 added to the logits, or NULL */
  const float* shared_gate_w;  /* [H] fp32 */
  const uint16_t* router_w3;   /* [3][E][H] bf16 from moe_prepack_router(); required by the grouped path */
} moe_layer;

/* Tile height (rows) that moe_forward uses for its block map. */
int32_t moe_block_m(void);

/* Entries a block map of tile height block_m may need: ceil(T*k/block_m) + E. */
int32_t moe_max_tiles(int32_t T, int32_t top_k, int32_t n_experts, int32_t block_m);

/* Split fp32 router weights [E][H] exactly into three bf16 planes
 * router_w3[0] + router_w3[1] + router_w3[2] == router_w (each plane keeps the
 * next 8 significant bits, truncating), so that bf16 matrix-core products of a
 * bf16 activation with the planes are exact and the router stays fp32-accurate.
 * A one-time weight preparation, like loading the checkpoint. */
moe_status moe_prepack_router(const moe_dims* d, const float* router_w, uint16_t* router_w3, void* stream);

/* Router logits: every token is scored against every routed expert (Lily page,
 * section "The architecture that forces the issue: MoE plus Gated DeltaNet").
 *   x [T][H] bf16 -> logits [T][E] fp32 = x . router_w^T (+ router_bias),
 *                    shared_logit [T] fp32 = x . shared_gate_w  (NULL to skip).
 * T == 1 reads router_w (fp32 vector ALU dot products); T > 1 needs
 * layer->router_w3 (bf16 matrix cores, fp32 accumulation).  Only the router
 * fields of `layer` are read. */
moe_status moe_router_logits(const moe_dims* d, const moe_layer* layer, const uint16_t* x, int32_t T,
                             float* logits, float* shared_logit, void* stream);

/* Top-k routing from logits: each token keeps its 8 best-scored experts (same section).
 *   logits [T][E] fp32 -> ids [T][k] int32: the k largest logits in descending
 *   order, equal logits (+0 == -0) ordered by the lower expert index;
 *   weights [T][k] fp32: softmax over all E logits restricted to the kept
 *   experts and renormalised to sum to 1, i.e. exp(l_j - l_0) / sum_j' exp(l_j' - l_0);
 *   if shared_logit and gate are both non-NULL: gate[T] = 1 / (1 + exp(-shared_logit)).
 * Deterministic.  Inputs must be finite. */
moe_status moe_route(const moe_dims* d, const float* logits, const float* shared_logit, int32_t T, int32_t* ids,
                     float* weights, float* gate, void* stream);

/* Device error word of a workspace (moe_forward's or moe_group's): enqueues a
 * copy of it on `stream`, synchronises the stream, stores the MOE_DEVERR_* bits
 * in *flags and, when clear != 0, zeroes the word (also stream-ordered and
 * waited for).  Blocks the calling thread; not for use under graph capture. */
moe_status moe_workspace_errors(void* workspace, size_t workspace_bytes, int32_t clear, int32_t* flags, void* stream);

/* Scratch bytes moe_group() needs for T tokens (the 256-byte header included). */
size_t moe_group_workspace_bytes(const moe_dims* d, int32_t T);

/* GPU-resident grouping of the T*k routed slots by expert: histogram and block
 * map never leave the GPU (Inside Lily page, section "Performance Gains and
 * Workload Patterns").  Flat slot f = t*k + j.
 *   counts   [E]      slots per expert (sum = T*k)
 *   offsets  [E+1]    exclusive prefix sum of counts, offsets[E] = T*k
 *   perm     [T*k]    slots grouped by expert; within an expert ascending f (stable)
 *   inv_perm [T*k]    inv_perm[perm[p]] = p
 *   block_map[max_tiles][2] (expert, first row) for every tile of block_m rows,
 *                     experts ascending; unused entries (-1, -1)
 *   n_tiles  [1]      number of used entries (never leaves the device)
 * max_tiles must be >= moe_max_tiles(T, k, E, block_m); 1 <= block_m <= 4096.
 * ids values must lie in [0, E): a slot whose id does not is skipped (its
 * inv_perm entry is -1) and MOE_DEVERR_EXPERT_ID is set in the workspace's
 * error word.  Bitwise deterministic. */
moe_status moe_group(const moe_dims* d, const int32_t* ids, int32_t T, int32_t block_m, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv_perm, int32_t* block_map, int32_t max_tiles,
                     int32_t* n_tiles, void* workspace, size_t workspace_bytes, void* stream);

typedef enum moe_epilogue {
  /* h[p][n] = bf16( silu(gate) * up ), gate/up = a_row(p) . W_gate_up[e]^T */
  MOE_EPI_SWIGLU_BF16 = 0,
  /* y[perm[p] / k][m] += row_weight[perm[p]] * (a_row(p) . W_down[e]^T)[m]   (fp32 atomics) */
  MOE_EPI_WEIGHTED_SCATTER_F32 = 1
} moe_epilogue;

/* Grouped GEMM over the tiles of a block map with int4 weights dequantised in
 * registers, tile by tile inside the GEMM (bf16 matrix cores, fp32
 * accumulation; Inside Lily page, section "Performance Gains and Workload
 * Patterns"; the weighted scatter-combine is the layer's combine of the k
 * expert outputs of a token, Lily page, section "The architecture that forces
 * the issue").  Routed experts only.
 *   a_row(p): a_rows_are_tokens = 1: row perm[p] / k of a [T][K] (token rows,
 *             gathered through the permutation); 0: row p of a [T*k][K]
 *             (rows already in grouped order).  K = H for SWIGLU, I otherwise.
 *   SWIGLU:  w = gate_up weights; out = h [T*k][I] bf16 in grouped order.
 *   SCATTER: w = down weights; row_weight [T*k] fp32 indexed by flat slot;
 *            out = y [T][H] fp32, accumulated into (the caller zeroes it
 *            first).  Accumulation order across experts is not fixed, so y is
 *            reproducible to fp32 rounding.
 * w->packed must hold the matrix-core layout of the routed experts' matrix
 * (MOE_MAT_GATE_UP for SWIGLU, MOE_MAT_DOWN otherwise): the grouped GEMMs read
 * only that layout (moe_prepack_q4), never the canonical arrays.
 * perm/offsets/block_map/n_tiles as produced by moe_group() with the same
 * block_m (the kernels trust them: expert ids in [0, E), rows inside [0, T*k));
 * 1 <= block_m <= moe_block_m(). */
moe_status moe_grouped_gemm_q4(const moe_dims* d, const moe_q4* w, int32_t epi /* moe_epilogue */, const uint16_t* a,
                               int32_t a_rows_are_tokens, const int32_t* perm, const int32_t* offsets,
                               const int32_t* block_map, const int32_t* n_tiles, int32_t max_tiles,
                               const float* row_weight, int32_t T, int32_t block_m, void* out, void* stream);

/* Scratch bytes moe_forward() needs for up to T_max tokens.  After the
 * 256-byte header (error word) come the hand-over words of the fused path (1-4
 * tokens): per-block counts of completed calls and tagged data words.  They
 * must be zero before a workspace's first fused call (allocate it
 * zero-filled); after that every fused call keeps them consistent, and the
 * grouped path never writes them. */
size_t moe_workspace_bytes(const moe_dims* d, int32_t T_max);

/* The fused layer that moe_forward runs for T tokens of these dims (T <= 4,
 * see moe_forward) launches *needed workgroups that hand data to each other,
 * so all of them must be resident on the device at once.  *resident is what
 * the current device holds of that kernel at once (compute units x workgroups
 * per unit).  moe_forward refuses the fused path with MOE_ERR_UNSUPPORTED when
 * resident < needed (a partitioned or CU-masked device).  Returns
 * MOE_ERR_UNSUPPORTED when (d, T) does not take the fused path and MOE_ERR_HIP
 * when the device cannot be queried.  The answer is kept per device. */
moe_status moe_fused_residency(const moe_dims* d, int32_t T, int32_t* needed, int32_t* resident);

/* The whole layer for T tokens: every token is scored against the routed
 * experts, the best k are kept and a shared expert runs on every token (Lily
 * page, section "The architecture that forces the issue: MoE plus Gated
 * DeltaNet"); routing histograms and block maps stay on the GPU and the int4
 * weights are rebuilt inside the grouped GEMMs (Inside Lily page, section
 * "Performance Gains and Workload Patterns"); one token runs as GEMV on the
 * vector ALUs (Lily page, section "Why Apple Silicon isn't just a smaller
 * datacenter GPU"):
 *   y[t] = bf16( sum_j w[t][j] * E_{ids[t][j]}(x[t]) + g[t] * E_shared(x[t]) ),
 *   E(x) = ( silu(x.Wg^T) * (x.Wu^T) ) . Wd^T with the SwiGLU product rounded to bf16.
 * T == 1 (and 2 <= T <= 4 with hidden <= 2048, inter and shared_inter <= 512,
 * k <= 8) runs the fused decode path: one launch for the whole layer
 * (vector-ALU GEMV on the canonical weights, fp32 router_w), whose workgroups
 * hand results to each other through words in the workspace (see
 * moe_workspace_bytes; T == 1 needs hidden <= 4096, inter and shared_inter <=
 * 1024).  Larger T runs router GEMM, top-k, grouping, the two grouped GEMMs on
 * the matrix cores (needs router_w3 and the packed weights of all four
 * matrices) and the combine;
 * the shared expert's tiles run in the same GEMM launches.  The down GEMM stores every
 * routed slot's output and the shared expert's output unweighted, as fp16
 * values with a power-of-two exponent per 64 columns (fp32's range; fp16's
 * 11-bit precision for every value within 2^28 of its 64-column chunk's
 * largest), and a final pass multiplies each of a token's k+1 entries by its
 * routing weight (the shared one by the gate) and sums them in slot order in
 * fp32, so y is bitwise reproducible.  The fused path keeps everything in
 * fp32 registers.  Inputs must be finite.
 * No host synchronisation anywhere.
 * Optional outputs (NULL to skip): logits_out [T][E], ids_out [T][k], w_out [T][k].
 * workspace_bytes must be >= moe_workspace_bytes(d, T). */
moe_status moe_forward(const moe_dims* d, const moe_layer* layer, const uint16_t* x, int32_t T, uint16_t* y,
                       float* logits_out, int32_t* ids_out, float* w_out, void* workspace, size_t workspace_bytes,
                       void* stream);

/* moe_forward for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The workspace is a device global of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends; nothing is allocated and no allocating library
 * routine is called.  The caller still passes the inputs and outputs, as for
 * moe_forward.  T whose moe_workspace_bytes(d, T) exceeds the scratch (for the
 * model's dims, T above about 600) returns MOE_ERR_WORKSPACE.  Every call on a
 * device shares that device's scratch: calls that overlap on one device (on
 * different streams, or from different threads) race and must not be made;
 * calls on one stream are ordered.  The scratch's device error word has no
 * reader: use moe_forward with an own workspace to inspect it. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
moe_status moe_forward_noalloc(const moe_dims* d, const moe_layer* layer, const uint16_t* x, int32_t T, uint16_t* y,
                               float* logits_out, int32_t* ids_out, float* w_out, void* stream);

/* The stages of moe_forward, in order.  Grouped path: router GEMM (partial sums over
 * K splits when T is small), top-k + tile histogram, grouping, gate/up grouped GEMM
 * (+ shared expert), down grouped GEMM writing the unweighted slot outputs
 * (+ shared expert), weighted combine to bf16.  Fused path (1-4 tokens, see
 * moe_forward): the whole layer runs as the ROUTER stage; the other stages are
 * empty. */
typedef enum moe_stage {
  MOE_STAGE_ROUTER = 0,
  MOE_STAGE_TOPK = 1,
  MOE_STAGE_GROUP = 2,
  MOE_STAGE_GATE_UP = 3,
  MOE_STAGE_DOWN = 4,
  MOE_STAGE_COMBINE = 5
} moe_stage;

/* moe_forward restricted to stages first..last (inclusive).  A stage reads
 * what the earlier stages left in `workspace`, so a range that does not start
 * at MOE_STAGE_ROUTER needs a previous call on the same workspace, inputs and
 * optional outputs.
 * moe_forward() is moe_forward_stages(..., MOE_STAGE_ROUTER, MOE_STAGE_COMBINE).
 * Lets a caller time one stage alone or interleave its own work between stages. */
moe_status moe_forward_stages(const moe_dims* d, const moe_layer* layer, const uint16_t* x, int32_t T, uint16_t* y,
                              float* logits_out, int32_t* ids_out, float* w_out, void* workspace,
                              size_t workspace_bytes, int32_t first, int32_t last, void* stream);

/* Host-side offsets and block map from per-expert counts (no GPU involved):
 * offsets[E+1] exclusive prefix sum, block_map[max_tiles][2] (expert, first
 * row) for every tile of block_m rows, experts ascending, unused entries
 * (-1, -1), *n_tiles used entries; the same values moe_group() computes on the
 * GPU.  All pointers are host memory.  MOE_ERR_INVALID_ARG for a negative
 * count, a sum past 2^31 or more tiles than max_tiles. */
moe_status moe_host_block_map(const int32_t* counts, int32_t E, int32_t block_m, int32_t max_tiles, int32_t* offsets,
                              int32_t* block_map, int32_t* n_tiles);

/* Host bytes moe_forward_host_routing() needs for T tokens. */
size_t moe_host_routing_bytes(const moe_dims* d, int32_t T);

/* moe_forward (grouped path) with the routing round trip through the host that the
 * pages removed (Inside Lily page, section "Key Optimizations at a Glance", GPU-resident
 * expert routing): after top-k the per-expert counts are copied to the
 * host, the stream is synchronised, offsets and block map are built on the
 * host (moe_host_block_map) and copied back, and the permutation, GEMMs and
 * combine follow as in moe_forward.  Same kernels and grouping, so y, ids and
 * weights are bitwise those of moe_forward.  Measures what the GPU-resident
 * grouping saves; it blocks the calling thread and cannot be captured into a
 * graph.  host_buf: host memory of moe_host_routing_bytes(d, T) bytes (pinned
 * memory keeps the copies asynchronous), reused across calls.  A T that
 * moe_forward runs on the fused path (1-4 tokens) is MOE_ERR_UNSUPPORTED. */
moe_status moe_forward_host_routing(const moe_dims* d, const moe_layer* layer, const uint16_t* x, int32_t T,
                                    uint16_t* y, int32_t* ids_out, float* w_out, void* workspace,
                                    size_t workspace_bytes, void* host_buf, size_t host_bytes, void* stream);

/* Grouped-query attention, one decode step (one query row per head) for B
 * sequences.  The model's full-attention layers have 16 query heads sharing 2
 * key/value heads (Lily page, section "The architecture that forces the
 * issue"); the "Inside Lily ..." page (section "Key Optimizations at a Glance")
 * names GQA packing, one load of each key/value row for all the query heads of
 * its group, among its optimisations.
 *   q [B][Hq][D] bf16 (4-byte aligned); k_cache, v_cache [B][Hkv][S][D] bf16 (16-byte aligned),
 *   S positions of capacity per sequence and head; seq_lens [B] int32 positions
 *   in use (values are clamped to [0, S]); out [B][Hq][D] bf16.
 *   Query head h reads key/value head h / (Hq / Hkv):
 *   out = sum_p softmax_p(scale * q . k_p) v_p over p < seq_lens[b], scores,
 *   softmax and sums in fp32 (the probabilities enter the weighted sum of
 *   value rows split into two bf16 parts, 16 significant bits), one bf16
 *   rounding; a sequence of length 0 gives zeros.  The positions are cut into ranges that run in parallel; their
 *   partial results are merged in range order, so out is reproducible.
 *   pack_heads = 1: a workgroup takes all Hq / Hkv query heads of a group and
 *   loads each key/value row once; pack_heads = 0: one query head per
 *   workgroup, each row loaded once per query head (the unpacked form, kept to
 *   measure what packing saves).
 * Supported: Hq % Hkv == 0, Hq / Hkv <= 8, D in {64, 128, 256}, 1 <= B <= 4096,
 * 1 <= S <= 2^22.  workspace (16-byte aligned) of at least
 * moe_gqa_decode_workspace_bytes(B, Hq, Hkv, D, S) bytes; 0 for an unsupported
 * shape. */
size_t moe_gqa_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S);
moe_status moe_gqa_decode_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                    const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t S,
                                    float scale, int32_t pack_heads, uint16_t* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* Human-readable name of a status ("MOE_ERR_UNKNOWN" for a value that is none);
 * message of the last failed check on this thread. */
const char* moe_status_str(int32_t status);
const char* moe_last_error_message(void);
/* hipError_t of the last failed launch on this thread (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
