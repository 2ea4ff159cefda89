/*
 * sgemm.h -- small-M decode GEMM and persistent per-layer projection chain on
 * AMD Instinct MI355X (gfx950).  C ABI of libsgemm.so.
 *
 * The operation (Fleet, "Hierarchical Task-based Abstraction for Megakernels
 * on Multi-Die GPUs", reading note: Summary, section 3f notation table and
 * section 4; restated for MI355X by the news item "ROCm Low-Latency-GEMM-
 * Kernel ... bis zu 1,79x auf Instinct MI355X", section "Was ist GEMM"):
 *
 *     Y[M,N] = X[M,K] . W[K,N]       bf16 inputs, fp32 accumulation,
 *                                    M = 1..64 (the decode batch),
 *                                    K and N in the thousands.
 *
 * Layouts (all dense, no padding):
 *   X  row-major [M][K] bf16            (row m at X + m*K)
 *   W  K-major   [N][K] bf16            (output column n is the contiguous run
 *                                        W + n*K, the layout the per-chiplet
 *                                        weight pointer base + k*(N/8)*K*2
 *                                        presupposes; nn.Linear's layout)
 *   Y  row-major [M][N] fp32 or bf16
 *
 * Ownership: the caller allocates and owns every device buffer (X, W, Y and the
 * workspace).  A plan owns only host-side metadata.  No call allocates device
 * memory; sgemm_topology_probe and sgemm_read_probe write into caller buffers.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 * sgemm_run and layerchain_run enqueue work and return; they never
 * synchronise.  Errors detected on the device (watchdog time-out, XCD mapping
 * mismatch) are latched in the workspace status word and reported by
 * sgemm_query_status.
 *
 * Errors: every call returns an sgemm_status; nothing throws across the ABI.
 * Argument errors are detected before anything is enqueued.
 */
#ifndef SGEMM_H
#define SGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sgemm_plan_s* sgemm_plan;

typedef enum {
  SGEMM_OK = 0,
  SGEMM_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, bad flag  */
  SGEMM_ERR_UNSUPPORTED = -2, /* valid but outside what is built (e.g. M>64)  */
  SGEMM_ERR_HIP = -3,         /* a HIP runtime call failed                    */
  SGEMM_ERR_TIMEOUT = -4,     /* a device-side bounded wait expired           */
  SGEMM_ERR_WORKSPACE = -5,   /* workspace too small / not initialised        */
  SGEMM_ERR_TOPOLOGY = -6     /* workgroups did not map onto the XCDs as a
                                 round-robin from some starting XCD          */
} sgemm_status;

enum { SGEMM_KIND_GEMM = 0, SGEMM_KIND_LAYERCHAIN = 1, SGEMM_KIND_DECODER = 2 };
enum { SGEMM_OUT_F32 = 0, SGEMM_OUT_BF16 = 1 };

/* Plan flags (bitwise OR). */
enum {
  SGEMM_F_FORCE_DOT2 = 1u << 0,  /* use the VALU dot2 path whatever M is (M < 16
                                    only in the chain)                          */
  SGEMM_F_FORCE_MFMA = 1u << 1,  /* use the MFMA path whatever M is             */
  SGEMM_F_W_CACHED = 1u << 2,    /* weight loads without the nontemporal hint    */
  SGEMM_F_SYNC_FLAT = 1u << 3,   /* chain: every workgroup publishes globally     */
  SGEMM_F_SYNC_AGENT = 1u << 4,  /* split-K: device-scope release/acquire instead
                                    of the XCD-local (same-L2) protocol          */
  SGEMM_F_STAMPS = 1u << 5,      /* chain: record per-workgroup stage timestamps  */
  SGEMM_F_WATCHDOG_TEST = 1u << 6, /* chain: spin budget of zero, to exercise the
                                      time-out path from the host               */
  SGEMM_F_W_SC1 = 1u << 7,       /* weight loads with sc1|nt (streaming)         */
  SGEMM_F_POLL_LEADER = 1u << 8, /* chain: one workgroup per XCD polls the global
                                    counter and raises a per-XCD flag that the
                                    XCD's other workgroups poll (default: every
                                    workgroup polls the global counter)         */
  SGEMM_F_MTILE_ITEMS = 1u << 9, /* GEMM, ablation: one window of T_M rows
                                    (problem field tm: 16, 32 or 64) per item,
                                    m-tile fastest, consecutive items on
                                    neighbouring waves, so the windows of a
                                    column block share its weights through the
                                    caches (Fleet reading note, section 3f,
                                    M-major window, T_M) instead of in
                                    registers; MFMA path, no K slices           */
  SGEMM_F_LAUNCH_PER_STAGE = 1u << 10, /* chain, ablation: one launch of the same
                                    kernel per projection stage, so the kernel
                                    boundary is the barrier between stages and
                                    no weights are prefetched across it; the
                                    results are bitwise those of one launch     */
  SGEMM_F_CHECK_PLACEMENT = 1u << 12, /* GEMM: every workgroup claims its (XCD,
                                    slot) pair in the workspace after its work
                                    and a pair claimed twice latches
                                    SGEMM_ERR_TOPOLOGY (Fleet reading note,
                                    section 3b: the runtime learns each
                                    workgroup's XCD from the hardware id).
                                    Costs 1.5-3 us per launch (a device-scope
                                    atomic round trip at the end), so it is
                                    opt-in; the chain always checks (once per
                                    launch).  Refused for the chain
                                    (SGEMM_ERR_UNSUPPORTED)                     */
  SGEMM_F_MSPLIT = 1u << 14,     /* GEMM, ablation: the m-tile items of
                                    SGEMM_F_MTILE_ITEMS in the M-split order --
                                    column block fastest, so neighbouring
                                    waves read different weights and no m-tile
                                    of a block shares them with another in time
                                    (Fleet reading note, section 7, Table 4 and
                                    its key findings: M-tile against M-split;
                                    section 3f, Eq.(1) with R = 1)              */
  SGEMM_F_KCHUNK = 1u << 13,     /* the K-chunked MFMA path: the eight waves of
                                    a workgroup share one block of tiles over a
                                    K split, X goes through LDS in 512-wide K
                                    chunks, double-buffered, so the split no
                                    longer has to fit the LDS (the news item on
                                    MI355X low-latency GEMM, techniques 2 and
                                    3; the Fleet reading note's missing
                                    wave-level K split, Limitations).  tn, when
                                    given, is 16 x the tiles per block (32, 48,
                                    64, 96 or 128); kslices must be 0 or 1 and waves
                                    0 or 8.  In the chain (an ablation, built
                                    for M = 17-32, else SGEMM_ERR_UNSUPPORTED):
                                    every stage on this path, the gate_up stage
                                    with whole (gate, up) tile pairs; tn fixes
                                    the tiles of the unpaired stages            */
  SGEMM_F_SCHEDULER = 1u << 11   /* chain, ablation: the per-XCD scheduler
                                    runtime (Fleet reading note, sections 3b
                                    and 5, the runtime layout figure of
                                    section 4, the per-worker ready-task id
                                    of section 11a, finding 4): slot 0
                                    of each XCD does no GEMM work; it polls
                                    the global counter of each event and then
                                    writes the next task id into the
                                    ready-task word of each of the XCD's 31
                                    workers, which poll only their own word.
                                    The other 31 slots share the stages'
                                    items.  Not combined with
                                    SGEMM_F_SYNC_FLAT or SGEMM_F_POLL_LEADER
                                    (SGEMM_ERR_UNSUPPORTED)                     */
};

/*
 * Problem description.
 *   kind = SGEMM_KIND_GEMM:       M, K, N, out_dtype.
 *   kind = SGEMM_KIND_LAYERCHAIN: M, n_layers, d_model, q_cols, d_ff.  Per layer
 *       (Fleet reading note, sections 3f and 7b: gate and up concatenated and
 *       SiLU-gated; one decoder layer's projections back to back):
 *         h1 = bf16(x . Wq^T)  h2 = bf16(h1 . Wo^T)  [g|u] = h2 . Wgu^T
 *         a = bf16(silu(g) * u)  x' = bf16(a . Wdown^T)
 *       with Wq [q_cols][d_model], Wo [d_model][q_cols], Wgu [2 d_ff][d_model]
 *       (g = rows 0..d_ff-1, u = rows d_ff..2 d_ff-1), Wdown [d_model][d_ff],
 *       all K-major.
 *   tn, splitk, waves, kslices: 0 lets the planner choose; otherwise they
 *       override the columns per wave tile, the K split count across
 *       workgroups, the waves per workgroup and (MFMA path) the K slices per
 *       item inside a workgroup (1, 2, 4 or 8; slices are reduced through LDS).
 */
typedef struct {
  int kind;
  int M, K, N;
  int out_dtype;
  int n_layers, d_model, q_cols, d_ff;
  unsigned flags;
  int tn, splitk, waves, kslices;
  int tm;  /* SGEMM_F_MTILE_ITEMS / SGEMM_F_MSPLIT: rows per item, T_M = 16, 32 or
              64 (0: 16).  Single GEMM with M > 64 on the large-tile path:
              rows of a workgroup tile, 64, 128 or 256 (0: the planner's);
              tn there is the tile's columns.  Tiles built (rows x columns):
              64 x 96, 128 x 96, 128 x 192 and 256 x 96 with four waves,
              twice the columns with eight; others are refused with
              SGEMM_ERR_UNSUPPORTED.  Must be 0 otherwise */
  /* kind = SGEMM_KIND_DECODER: M, n_layers, d_model, d_ff and these (q_cols is
     0 or n_heads * head_dim).  Built: n_heads = 4 n_kv_heads, head_dim = 128,
     ctx + 1 <= 4096 (64 chunks of 64 positions), M <= 64. */
  int n_heads, n_kv_heads, head_dim; /* query heads, key/value heads, head dim */
  int ctx;                           /* cached positions T per sequence          */
} sgemm_problem;

/*
 * Build a plan for device `device` (a HIP ordinal).  Validates the problem,
 * chooses the path (dot2 for M < 16, MFMA for M >= 16, unless forced), the
 * per-XCD column partition, tile widths, split-K count and workspace layout.
 * *workspace_bytes receives the size of the device workspace the runs need
 * (>= 4 KiB).  Shape rules: 1 <= M <= 256 for the single GEMM and
 * 1 <= M <= 64 for the chain and the decoder; K >= 8, K % 8 == 0; N >= 1;
 * every operand below 2 GiB.  Returns SGEMM_ERR_INVALID_ARG or
 * SGEMM_ERR_UNSUPPORTED without creating a plan when they are violated.
 * A single GEMM with M = 65..256 (the compute-leaning regime: the scope of
 * the FlyDSL news item's K-split and multi-stage LDS pipeline, and the batch
 * sizes at which the Fleet reading note reports its megakernel falling
 * behind, Limitations) runs on the large-tile MFMA path: a workgroup of four
 * or eight waves (2 x 2 or 2 x 4) owns a tile of 64-256 rows and 96-384
 * columns over a K split; each 64-wide K step's X and W blocks are fetched a
 * few steps ahead by whole-line register loads and written to one of two LDS
 * buffers, from which every wave reads its MFMA fragments.  By default eight
 * waves over 64 x 192 tiles up to 128 rows and 128 x 192 above; the same
 * path, with four waves over 64 x 96 tiles, also takes M = 49..64 when N or
 * K is at least 12288.  With SGEMM_F_KCHUNK it runs on the K-chunked MFMA path in 64-row
 * m-blocks instead.  On both, the m-blocks of a column block are
 * neighbouring items that an XCD's workgroups take round-robin, so they
 * share the block's weight lines through that XCD's L2 (the M-major window,
 * section 3f, Eq.(1)); on the large-tile path the weights are then loaded
 * with the default cache policy (nontemporal with one m-block), which keeps
 * the lines in L2 for the later readers.  There SGEMM_F_FORCE_DOT2,
 * SGEMM_F_FORCE_MFMA, SGEMM_F_MTILE_ITEMS, SGEMM_F_MSPLIT and SGEMM_F_W_SC1
 * are refused with SGEMM_ERR_UNSUPPORTED, SGEMM_F_W_CACHED too on the
 * K-chunked path (its kernels load weights nontemporally only, at any M),
 * and so are kslices above 1 and, on the large-tile path, waves other than
 * 0, 4 or 8.
 *
 * Environment, read here (for experiments and calibration):
 *   SGEMM_TN, SGEMM_SPLITK, SGEMM_WAVES, SGEMM_KSLICES: used for the problem
 *       fields tn, splitk, waves, kslices when those are 0;
 *   SGEMM_CHAIN_S, SGEMM_CHAIN_KSL, SGEMM_CHAIN_WPI: "q,o,gate_up,down", the
 *       split count, K slices and waves per item of each chain stage
 *       (0 = the planner's choice);
 *   SGEMM_CHAIN_COST: "alpha,x_gbps,split_us,fin_us_kb,ksl_us", the chain
 *       planner's cost constants;
 *   SGEMM_WATCHDOG_S: seconds a chain stage may wait for its producer before
 *       the run stops with SGEMM_ERR_TIMEOUT (default 5, at most 3600);
 *   SGEMM_LT (default 1): 0 runs M = 65..256 on the K-chunked path instead
 *       of the large-tile one;
 *   SGEMM_LT_MIN_M (default 65): the fewest rows (at least 16) that take the
 *       large-tile path; below 65 it replaces the MFMA paths from that M on;
 *   SGEMM_DOT2_RR, SGEMM_MFMA_RR, SGEMM_KC_RR, SGEMM_CHAIN_RR (default 1): 0
 *       gives each workgroup a contiguous range of its XCD's items instead of
 *       every 32nd item (single-GEMM dot2 and MFMA plans without splits,
 *       K-chunked and large-tile plans with several m-blocks, chain stages);
 *   SGEMM_CHAIN_WPF (default 0): weight steps that each chain dot2 stage
 *       loads into LDS before its wait for X;
 *   SGEMM_CHAIN_GCOPIES (8 or 1, default 8): copies of each chain and
 *       decoder counter, one per XCD or one for all;
 *   SGEMM_ATTN_SLICES (1..8): the decoder's attention workgroup slices per
 *       (sequence, key/value head) pair (default: the planner's).
 * A malformed value makes the call return SGEMM_ERR_INVALID_ARG.
 */
int sgemm_plan_create(const sgemm_problem* problem, int device, sgemm_plan* out,
                      size_t* workspace_bytes);

/* Release a plan (host memory only).  NULL is accepted. */
int sgemm_plan_destroy(sgemm_plan plan);

/*
 * Zero a workspace of plan's size with a fill kernel on `stream`.  Must be
 * called once after allocation (a zero-filled allocation is equivalent).
 * Afterwards the runs keep it consistent themselves (split-K tile counters are
 * reset by their last arriver; chain counters by the last workgroup to
 * finish).  A workspace belongs to one plan and must not be used by two runs
 * that can overlap in time.
 */
int sgemm_workspace_init(sgemm_plan plan, void* workspace, void* stream);

/*
 * Y = X . W (kind GEMM).  X [M][K] bf16, W [N][K] bf16, Y [M][N] (fp32 or bf16
 * as planned); all device pointers, 16-byte aligned.  Enqueues one kernel on
 * `stream` and returns.  SGEMM_ERR_UNSUPPORTED when the plan's device is not
 * a 256-CU gfx950 (sgemm_device_check).  With SGEMM_F_CHECK_PLACEMENT each
 * launch also checks on the device that its 256 workgroups covered every
 * (XCD, slot) pair exactly once; a violation latches SGEMM_ERR_TOPOLOGY for
 * sgemm_query_status.
 */
int sgemm_run(sgemm_plan plan, const void* X, const void* W, void* Y, void* workspace,
              void* stream);

/*
 * sgemm_run without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The split-K counters and partials live in a 32 MiB
 * array of the library's own (a static device array, one copy per GPU, held
 * until the process ends; its address is looked up once per device).  Same
 * kernels, plan and results as sgemm_run.
 *   Limits: the plan's split-K counters must fit 1 MiB and its partials
 *   32 MiB - 1 MiB - 256 B, else SGEMM_ERR_WORKSPACE (every decode
 *   projection shape up to M = 256 fits; the largest, 256 x 4096 x 6144 in
 *   four splits, needs 24 MiB).
 *   SGEMM_F_CHECK_PLACEMENT plans are refused (SGEMM_ERR_UNSUPPORTED): no
 *   status word is read back from the shared array.
 *   Concurrency: every call on a GPU uses that GPU's one array, so calls
 *   that can overlap in time on the same GPU (two streams, two threads) race
 *   and give wrong results; serialise them.  Calls in stream order are safe:
 *   each run leaves the counters at zero for the next.
 *   Other errors as sgemm_run.  Allocates nothing (no hipMalloc, no
 *   allocating library call).
 */
int sgemm_run_noalloc(sgemm_plan plan, const void* X, const void* W, void* Y, void* stream);

/*
 * The whole layer chain in one persistent launch (kind LAYERCHAIN).
 * X0 [M][d_model] bf16 device pointer.  Wq, Wo, Wgu, Wdown are HOST arrays of
 * n_layers DEVICE pointers each (layouts above).  Y_f32 [M][d_model] receives
 * the last layer's down projection before rounding; Y_bf16 (may be NULL) its
 * bf16 rounding.  Intermediate activations stay in the workspace (see
 * sgemm_chain_buffer).  Enqueues one kernel and returns.
 *
 * Residency: the launch is a persistent grid of one workgroup per CU (256),
 * whose stages wait for each other, so it needs every one of its workgroups
 * resident at once.  Work running concurrently on the GPU (another stream)
 * delays it until CUs free up; two chain launches overlapping in time can
 * each hold CUs the other waits for, and then both end after the watchdog
 * budget (SGEMM_WATCHDOG_S) with SGEMM_ERR_TIMEOUT latched in the workspace.
 * Run chains on one stream, or serialise them.
 */
int layerchain_run(sgemm_plan plan, const void* X0, const void* const* Wq,
                   const void* const* Wo, const void* const* Wgu, const void* const* Wdown,
                   float* Y_f32, void* Y_bf16, void* workspace, void* stream);

/*
 * The whole decoder layer, all layers in one persistent launch (kind DECODER;
 * Fleet reading note, TL;DR and Summary: about seven operators per layer of
 * a Qwen3-8B-shaped decoder, all inside one megakernel; section 1: grouped-
 * query attention with 32 query and 8 key/value heads).  Per layer l, on the
 * residual stream x (X0 for layer 0):
 *   n1 = bf16(rmsnorm(x) * w_attn)            rmsnorm(v) = v / sqrt(mean(v^2) + 1e-6)
 *   [q|k|v] = bf16(n1 . Wqkv^T)               q: n_heads x head_dim, k, v: n_kv_heads x head_dim
 *   o  = bf16(attention)                       query head h reads key/value head h / 4 over the
 *                                              ctx cached positions and the new k, v (position ctx):
 *                                              sum_t softmax_t(q_h . k_t / sqrt(head_dim)) v_t
 *   x1 = bf16(x + o . Wo^T)
 *   a  = bf16(silu(g) * u), [g|u] = bf16(rmsnorm(x1) * w_mlp) . Wgu^T
 *   x' = bf16(x1 + a . Wdown^T)               (the last layer's also in fp32, Y_f32)
 * Pointers (device, 16-byte aligned):
 *   X0 [M][d_model] bf16; w_norm [n_layers][2][d_model] bf16 (w_attn, w_mlp);
 *   Wqkv, Wo, Wgu, Wdown: HOST arrays of n_layers device pointers, K-major
 *     [q + 2 kv][d_model], [d_model][q], [2 d_ff][d_model], [d_model][d_ff]
 *     (q = n_heads head_dim, kv = n_kv_heads head_dim; rows of Wqkv: q, then k, then v);
 *   K_cache, V_cache [n_layers][M][n_kv_heads][ctx][head_dim] bf16 (may be NULL when ctx = 0);
 *   Y_f32 [M][d_model]; Y_bf16 [M][d_model] or NULL.
 * The caches are read only: the new token's k and v of layer l are left in
 * the workspace (sgemm_chain_buffer which = 0, columns q .. q + 2 kv) for
 * the caller to append.  Intermediates: sgemm_chain_buffer which = 0 qkv,
 * 1 o, 2 x1, 3 a, 4 x'.  Errors and residency as layerchain_run.
 */
int decoder_run(sgemm_plan plan, const void* X0, const void* w_norm, const void* const* Wqkv,
                const void* const* Wo, const void* const* Wgu, const void* const* Wdown,
                const void* K_cache, const void* V_cache, float* Y_f32, void* Y_bf16, void* workspace,
                void* stream);

/*
 * Where the chain keeps an intermediate activation in the workspace:
 * which = 0 h1 [M][q_cols], 1 h2 [M][d_model], 2 a [M][d_ff], 3 x' [M][d_model]
 * (all bf16, row-major) of layer `layer`; for a decoder plan which = 0 qkv
 * [M][q + 2 kv], 1 o [M][q], 2 x1 [M][d_model], 3 a [M][d_ff], 4 x' [M][d_model].
 * Valid after the run has completed.
 */
int sgemm_chain_buffer(sgemm_plan plan, int layer, int which, size_t* offset, size_t* bytes);

/*
 * Synchronise `stream`, read and clear the workspace status word and return the
 * first device-side error latched since the last query (SGEMM_OK if none).
 */
int sgemm_query_status(sgemm_plan plan, void* workspace, void* stream);

/* Human-readable name of a status code (static storage). */
const char* sgemm_status_string(int status);

/*
 * JSON description of the plan (path, tiles, split-K, waves, grid, workspace
 * layout) written into buf (NUL-terminated, truncated to len).  Returns the
 * length needed.
 */
int sgemm_plan_describe(sgemm_plan plan, char* buf, size_t len);

/*
 * Whether `device` (a HIP ordinal) is what the kernels are built for: a gfx950
 * device exposing 256 CUs (8 XCDs of 32, one partition), the layout the
 * per-XCD column partition and the one-workgroup-per-CU grid assume (Fleet
 * reading note, section 3b: 8 XCDs of 32 CUs, each with its own L2; the
 * news item on MI355X low-latency GEMM: gfx950 with 256 CUs).  Queries the
 * device properties once and caches the answer.  sgemm_run and
 * layerchain_run make the same check before their first launch on a device.
 * Returns SGEMM_OK, SGEMM_ERR_UNSUPPORTED (another architecture or partition
 * mode), SGEMM_ERR_INVALID_ARG (device < 0 or >= 64) or SGEMM_ERR_HIP (the
 * query failed, e.g. no such device; not cached).
 */
int sgemm_device_check(int device);

/*
 * Topology probe: launch n_wg workgroups of one wave; workgroup i writes the
 * XCC id it ran on (the HW_REG_XCC_ID field) to xcc_out[i] (device int array
 * of n_wg entries).  Enqueues on `stream`; used to confirm the round-robin
 * workgroup-to-XCD dispatch the per-XCD partition relies on (Fleet reading
 * note, section 3b: default dispatch spreads workgroups round-robin over the
 * XCDs, and the runtime reads the hardware id to learn its XCD).  The
 * starting XCD varies between launches (graph launches move it), so the
 * kernels take their XCD from the hardware id and their slot from i / 8.
 */
int sgemm_topology_probe(int* xcc_out, int n_wg, void* stream);

/*
 * Read probe: the attainable-bandwidth reference for the weight stream (the
 * decode GEMM moves its 2*K*N weight bytes from HBM once, Fleet reading note,
 * section 2b roofline; this kernel only reads).  Launches `grid` workgroups
 * of 512 threads (grid a multiple of 8, 8..4096) that read `bytes` bytes at
 * `src` (device, 16-byte aligned, bytes a multiple of 16 and below 2 GiB) with
 * 16-byte nontemporal loads and xor all its 32-bit words into *sink (device,
 * 4-byte aligned; the caller zeroes it first if it checks the value).
 *   pattern 0: grid-stride order;
 *   pattern 1: the decode GEMM's order (XCD x reads the x-th eighth, each
 *              wave a contiguous share of it).
 * Enqueues on `stream`; returns SGEMM_ERR_INVALID_ARG for a bad argument
 * before enqueuing anything.
 */
int sgemm_read_probe(const void* src, size_t bytes, int pattern, unsigned* sink, int grid, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SGEMM_H */
