/*
 * tlsync.h — C ABI of the tile-level synchronised GEMM-chain library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library runs a chain of two dependent tiled contractions in ONE
 * persistent kernel launch: every workgroup takes work items from a global
 * atomic counter, producer tiles first, and a consumer tile starts as soon as
 * the particular producer tiles it reads are complete, instead of waiting at
 * a kernel boundary.  This is the fine-grained synchronisation of dependent
 * kernels of "A Framework for Fine-Grained Synchronization of Dependent GPU
 * Kernels" (Jangda et al., arXiv 2305.13450; below "the cuSync paper"),
 * sections "Fine-Grained Synchronization using cuSync" and "Synchronization
 * Policies", and, as an alternative handoff, the sentinel protocol of the
 * CUDA Programming Guide, 4.6 "Fine-Grained Synchronization" (below "the
 * sentinel guide"), 4.6.4 "Protocol".
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Tensor arguments are DEVICE pointers on the current HIP device, owned by
 *   the caller, contiguous (row-major / NHWC / [B,heads,S,d] as stated) and
 *   16-byte aligned.  Inputs are only read; outputs are fully overwritten.
 *   The library never frees a caller pointer.
 * - Element type is fp16 (IEEE binary16) unless an _ex call selects another
 *   supported dtype; accumulation is fp32; each stored value is rounded once,
 *   to nearest-even.
 * - Calls are ASYNCHRONOUS: they return after enqueueing work on the stream
 *   (NULL = the legacy default stream of the current device).  Device-side
 *   failures (a watchdog expiry) are reported by chain_sync() or
 *   chain_workspace_status().  With the environment variable TLSYNC_SYNC=1
 *   every call synchronises and returns the device status itself.
 * - No function throws, aborts or prints; errors are returned as negative
 *   chain_status codes and leave outputs unspecified.
 * - Concurrent calls that share a workspace (including the library-owned
 *   one of a device) must be ordered on one stream; overlapping calls race.
 */
#ifndef TLSYNC_H
#define TLSYNC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
typedef int chain_status;
#define CHAIN_OK            0
#define CHAIN_EINVAL       (-1) /* null/misaligned pointer, non-positive or inconsistent size */
#define CHAIN_EUNSUPPORTED (-2) /* shape not a multiple of an available tile, dtype or policy
                                   not valid for this chain */
#define CHAIN_EHIP         (-3) /* a HIP runtime call failed; see chain_last_hip_error() */
#define CHAIN_ETIMEOUT     (-4) /* a device wait exceeded its poll limit; see chain_last_timeout() */
#define CHAIN_ENOMEM       (-5) /* workspace allocation failed or caller workspace too small */
#define CHAIN_ESCRATCH     (-6) /* chain_mlp_noalloc: the call needs more workspace than the
                                   library's static scratch array holds (64 MiB) */

/* ---- sync policies (cuSync paper, "Synchronization Policies"; sentinel
 *      guide 4.6.4) ---------------------------------------------------------- */
#define CHAIN_STREAM_SERIAL     0 /* baseline: producer kernel, then consumer kernel, ordered by the
                                     stream (cuSync paper, "Stream Synchronization") */
#define CHAIN_TILESYNC          1 /* one flag per producer tile; a consumer tile waits on each producer
                                     tile of its row just before its K-loop enters that tile */
#define CHAIN_ROWSYNC           2 /* one counter per producer tile row; a consumer tile waits once for
                                     the whole row */
#define CHAIN_CONV2D_TILESYNC   3 /* conv chain only: a consumer pixel tile waits on the producer tiles
                                     covering its 3x3 halo (halo-aware reading of Conv2DTileSync) */
#define CHAIN_SENTINEL          4 /* MLP and conv chains: intermediate pre-filled with 0xFFFF (a NaN);
                                     the consumer re-polls any loaded element still holding it */
#define CHAIN_STRIDEDSYNC       5 /* self-attention chain: the first GEMM's tiles `heads` columns
                                     apart (one head's three slices) share one counter that the
                                     fused dot product waits on once (cuSync paper, paragraph
                                     StridedSync); the second GEMM waits per head (TileSync) */

/* ---- element types and activations ---------------------------------------- */
#define CHAIN_F16   0
#define CHAIN_BF16  1 /* chain_mlp: X, W1, W2, Y and the intermediate in bf16 (fp32
                         accumulation; tile configurations 0, 1, 6, 7, 9, 12 and 17 of
                         chain_tile_cfg_info, the ones the automatic plan picks; others
                         CHAIN_EUNSUPPORTED); chain_conv: X, Wa, Wb, Y and the
                         intermediate in bf16 (conv configurations 0, 3, 4 and 9, the
                         automatic ones and 4; others CHAIN_EUNSUPPORTED); chain_attn: Q, K, V, the scores
                         and O in bf16 (P enters the P.V product in bf16);
                         chain_selfattn: X, Wqkv, W2, XQKV, XDot and Y in bf16 (P enters
                         the second product in bf16) */

#define CHAIN_ACT_GELU_ERF   0 /* 0.5 x (1 + erf(x / sqrt 2)), the MLP default */
#define CHAIN_ACT_GELU_TANH  1 /* tanh approximation of GeLU */
#define CHAIN_ACT_NONE       2 /* identity (diagnostics) */
#define CHAIN_ACT_RELU       3 /* x < 0 ? 0 : x, the conv default */

/* ---- work orders ------------------------------------------------------------
 * Every order hands out all producer tiles before any consumer tile that
 * reads them, which is what makes the persistent chain deadlock-free. */
#define CHAIN_ORDER_XCD         0 /* default: one queue per XCD; queue q holds the tile columns of
                                     slab q (each weight panel is read by one XCD), row-major
                                     (conv: row slabs); producers of all queues, then consumers;
                                     idle XCDs steal.  The attention and conv chains, the
                                     MLP chain at M <= 128 and the self-attention chain at
                                     M >= 1024 run this default as CHAIN_ORDER_ROW_MAJOR
                                     (measured faster there) */
#define CHAIN_ORDER_ROW_MAJOR   1 /* one global counter: producer tiles row-major, then consumer
                                     tiles row-major (the cuSync paper's RowMajor order) */
#define CHAIN_ORDER_INTERLEAVED 2 /* one global counter: producer row r, then the consumer rows whose
                                     last producer row is r - 1 (MLP and attention: consumer row
                                     r - 1; conv: the rows whose 3x3 halo ends in producer row
                                     r - 1); consumer rows that read the last producer row follow
                                     it */
#define CHAIN_ORDER_COL_MAJOR   3 /* one global counter: producer tiles column by column, then
                                     consumer tiles column by column (cuSync paper, "Tile
                                     Processing Order": column major) */
#define CHAIN_ORDER_STRIDED     4 /* one global counter: producer tiles row by row, the columns of a
                                     row visited with stride s = order_stride (c, c+s, c+2s, ...,
                                     then c+1, ...), then consumer tiles the same way ("Tile
                                     Processing Order": strided row major) */
/* The tile grid an order walks: MLP rows of BM tokens x (column tiles x K
 * splits); conv pixel tiles x (channel tiles x K splits); attention (batch,
 * head) pairs x row blocks of 128 queries.  The conv pair at 64 output
 * channels has one column, where column-major and strided equal row-major. */

/* Extended MLP call.  Computes Z = act(X W1) (stored, rounded, NaN -> 0x7E00)
 * and Y = Z W2 with X:[M,H], W1:[H,F], W2:[F,H], Z:[M,F], Y:[M,H] row-major.
 * cuSync paper, section "GPT Models", Fig. "Architecture of two building
 * blocks of GPT models" (a).  Unused fields must be zero; a zeroed field
 * selects the default. */
typedef struct chain_mlp_args {
    const void* X;            /* [M,H] */
    const void* W1;           /* [H,F] */
    const void* W2;           /* [F,H] */
    void*       Y;            /* [M,H] output */
    int64_t     M, H, F;      /* M >= 1 (ragged M allowed); H, F multiples of 64 */
    int32_t     policy;       /* CHAIN_STREAM_SERIAL | TILESYNC | ROWSYNC | SENTINEL */
    int32_t     dtype;        /* CHAIN_F16 or CHAIN_BF16 */
    int32_t     act;          /* CHAIN_ACT_* (default GELU_ERF) */
    int32_t     tile_cfg;     /* 0 = automatic; k > 0: configuration k-1 of chain_tile_cfg_info() */
    void*       stream;       /* hipStream_t, NULL = default stream */
    void*       workspace;    /* NULL = library-owned per-device workspace */
    size_t      workspace_bytes;
    void*       z_out;        /* optional caller buffer [M,F] for the intermediate; NULL = workspace */
    float*      z_debug_f32;  /* optional [M,F] fp32 activation before rounding (slow, diagnostics) */
    uint64_t    order_seed;   /* 0 = the order's natural sequence; else a seeded permutation inside
                                 each group of the order (queue and phase, or row group) */
    int32_t     order;        /* CHAIN_ORDER_* */
    int32_t     grid;         /* 0 = automatic (CUs x occupancy); else persistent workgroups */
    uint32_t    poll_limit;   /* 0 = default; max polls of one wait before CHAIN_ETIMEOUT */
    int32_t     debug_skip_producer; /* 0 = none; k > 0: producer tile k-1 never posts (tests) */
    uint32_t    debug_delay;  /* 0 = none; else producers sleep a tile-dependent time before
                                 storing (race tests) */
    int32_t     split_k1;     /* K splits of a producer tile: 0 = automatic, 1 = none, s > 1:
                                 s splits (s must divide H / BK); deterministic reduction */
    int32_t     split_k2;     /* the same for consumer tiles (s must divide F / BK) */
    /* Sentinel buffer rotation (FGS 4.6.4.5 Buffer Reuse), CHAIN_SENTINEL only.
     * z_ring holds ring_slots intermediate buffers [M,F] back to back (16-byte
     * aligned, caller-owned, no z_out with it).  The call with ring_index i
     * consumes slot i % ring_slots and, inside the same launch, refills slot
     * (i + 1) % ring_slots with the sentinel, so no fill precedes the next
     * call.  i = 0 first fills slot 0 on the stream (priming).  Calls on one
     * ring must run in index order (one stream, or ordered); the intermediate
     * of call i stays in its slot until call i + ring_slots - 1 starts.  A call
     * that times out still leaves the next slot filled.  NULL = no ring: the
     * workspace intermediate is filled before every sentinel call. */
    void*       z_ring;
    int32_t     ring_slots;   /* 2..16 with z_ring, else ignored */
    uint32_t    ring_index;   /* sequence number of this call on the ring, from 0 */
    /* Optional per-item trace (measurement, not on the cuSync pages): NULL = off.
     * Otherwise a caller-owned, 16-byte aligned array of trace_capacity
     * chain_trace_rec; work item i (producer items first, K splits adjacent,
     * as chain_mlp_plan counts them) writes record i when it completes.
     * Records of items that did not run (a wait expired) are left as they
     * were.  trace_capacity below the call's work items is CHAIN_EINVAL. */
    void*       trace;
    uint32_t    trace_capacity;
    int32_t     order_stride; /* column stride of CHAIN_ORDER_STRIDED; 0 = 2 */
} chain_mlp_args;

/* One trace record (32 bytes).  Times are ticks of the GPU's constant-rate
 * realtime counter; chain_trace_clock_khz() gives its rate. */
typedef struct chain_trace_rec {
    uint32_t item;      /* work item index */
    uint16_t wg;        /* persistent workgroup that ran it */
    uint16_t hw;        /* XCD << 8 | shader engine << 5 | SH << 4 | CU */
    uint64_t t_start;   /* item taken from the scheduler */
    uint64_t t_ready;   /* its first dependency wait returned (t_start without one; for
                           CHAIN_SENTINEL the per-chunk re-polls are not counted) */
    uint64_t t_end;     /* item finished */
} chain_trace_rec;

/* Rate of the trace clock of the current device in kHz (hipDeviceAttributeWallClockRate). */
chain_status chain_trace_clock_khz(int* khz);

/* North-star form: fp16, GeLU(erf), automatic tile, library workspace,
 * default stream.  Returns CHAIN_OK once the chain is enqueued. */
chain_status chain_mlp(const void* X, const void* W1, const void* W2, void* Y,
                       int64_t M, int64_t H, int64_t F, int policy);
chain_status chain_mlp_ex(const chain_mlp_args* a);
/* Bytes of workspace one MLP call of this shape needs (0 on invalid input). */
size_t chain_mlp_workspace_bytes(int64_t M, int64_t H, int64_t F, int policy,
                                 int dtype, int tile_cfg);

/* Allocation-free form of chain_mlp_ex, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a static device array of the
 * library (64 MiB per device, held until the process ends) instead of a
 * caller buffer or the library-owned hipMalloc'd one: this call allocates
 * nothing on the device or through any allocating library routine.  Its first
 * call on a device clears the array's control and flag regions with a fill
 * kernel on a->stream.  Arguments as chain_mlp_ex, except: a->workspace must
 * be NULL (CHAIN_EINVAL); the work order must need no order table (order
 * CHAIN_ORDER_XCD or CHAIN_ORDER_ROW_MAJOR, order_seed 0; others
 * CHAIN_EUNSUPPORTED); a call whose workspace (chain_mlp_workspace_bytes)
 * exceeds the array returns CHAIN_ESCRATCH.  The intermediate lives in the
 * array unless z_out is given.  Every call on a device shares that device's
 * array, which keeps the last call's contents: calls that overlap on one
 * device race (order them on one stream).  Device status (a watchdog expiry)
 * is read with chain_noalloc_status. */
chain_status chain_mlp_noalloc(const chain_mlp_args* a);
/* chain_workspace_status for the static array of the current device. */
chain_status chain_noalloc_status(void* stream);

/* Conv pair, implicit GEMM: Z = ReLU(conv3x3(X, Wa)) (stored fp16), then
 * Y = conv3x3(Z, Wb).  X:[N,Hh,Ww,C], Z:[N,P,Q,K], Y:[N,P,Q,K] NHWC; Wa:[R,S,C,K],
 * Wb:[R,S,K,K] RSCK.  cuSync paper, section "ResNet" and the Table of ResNet-38
 * conv pairs; Conv2DTileSync in "Synchronization Policies".  This build
 * supports R = S = 3, pad = 1, stride = 1, C and K multiples of 64. */
typedef struct chain_conv_args {
    const void* X;
    const void* Wa;
    const void* Wb;
    void*       Y;
    int32_t     N, Hh, Ww, C, K, R, S, pad, stride;
    int32_t     policy;       /* STREAM_SERIAL | CONV2D_TILESYNC (TILESYNC is read as it) |
                                 ROWSYNC | SENTINEL */
    int32_t     dtype;        /* CHAIN_F16 or CHAIN_BF16 */
    int32_t     act;          /* 0 (the default) is read as CHAIN_ACT_RELU for conv */
    int32_t     tile_cfg;     /* 0 = automatic; k > 0: conv configuration k-1 */
    void*       stream;
    void*       workspace;
    size_t      workspace_bytes;
    void*       z_out;        /* optional [N,P,Q,K] intermediate */
    float*      z_debug_f32;  /* optional [N*P*Q,K] fp32 activation before rounding (diagnostics) */
    uint64_t    order_seed;
    int32_t     order;
    int32_t     grid;
    uint32_t    poll_limit;
    int32_t     debug_skip_producer; /* 0 = none; k > 0: producer tile k-1 never posts */
    uint32_t    debug_delay;
    int32_t     split_k1;     /* K splits of a producer tile: 0 = automatic, 1 = none, s > 1:
                                 s splits (s must divide R*S*C / 64); deterministic reduction */
    int32_t     split_k2;     /* the same for consumer tiles (s must divide R*S*K / 64) */
    void*       z_ring;       /* sentinel ring of [N,P,Q,K] intermediates, as in chain_mlp_args */
    int32_t     ring_slots;
    uint32_t    ring_index;
    void*       trace;        /* optional per-item trace, as in chain_mlp_args (items as
                                 chain_conv_plan counts them: producer tiles x split_k1, then
                                 consumer tiles x split_k2) */
    uint32_t    trace_capacity;
    int32_t     order_stride; /* column stride of CHAIN_ORDER_STRIDED; 0 = 2 */
    int32_t     debug_first_skip; /* test knob, 0 or 1: with the default order a launch's
                                     first items come from eight per-XCD counters; 1 makes
                                     workgroups with an odd block index take none, leaving
                                     their share to the sweep that runs before the first
                                     consumer item */
} chain_conv_args;

chain_status chain_conv(const void* X, const void* Wa, const void* Wb, void* Y,
                        int N, int Hh, int Ww, int C, int K, int R, int S,
                        int pad, int stride, int policy);
chain_status chain_conv_ex(const chain_conv_args* a);
size_t chain_conv_workspace_bytes(int N, int Hh, int Ww, int C, int K, int R, int S,
                                  int pad, int stride, int policy, int dtype, int tile_cfg);

/* Attention-score chain per (batch, head): Sc = fp16(scale Q K^T) (stored),
 * O = softmax_rows(Sc) V, softmax in fp32 over the key axis, no mask or
 * dropout.  Q, K, V, O: [B, heads, S, d] contiguous.  cuSync paper, section
 * "GPT Models", Fig. "Architecture of two building blocks of GPT models" (b),
 * synchronised by rows (RowSync).  This build supports d = 128 and S a
 * multiple of 128. */
typedef struct chain_attn_args {
    const void* Q;
    const void* K;
    const void* V;
    void*       O;
    int32_t     B, heads, S, d;
    float       scale;
    int32_t     policy;       /* STREAM_SERIAL | ROWSYNC | TILESYNC */
    int32_t     dtype;        /* CHAIN_F16 or CHAIN_BF16 */
    int32_t     tile_cfg;
    void*       stream;
    void*       workspace;
    size_t      workspace_bytes;
    void*       s_out;        /* optional [B,heads,S,S] buffer for the scores */
    uint64_t    order_seed;
    int32_t     order;
    int32_t     grid;
    uint32_t    poll_limit;
    int32_t     debug_skip_producer; /* 0 = none; k > 0: producer item (a score row block
                                        against every key block) k-1 never posts */
    uint32_t    debug_delay;
    int32_t     ring_slots;   /* sentinel ring of [B,heads,S,S] score buffers in s_ring, as in */
    uint32_t    ring_index;   /* chain_mlp_args (z_ring): CHAIN_SENTINEL only, no s_out with it */
    void*       s_ring;
    void*       trace;        /* optional per-item trace, as in chain_mlp_args: the
                                 B*heads*S/128 producer row blocks, then as many consumer
                                 row blocks */
    uint32_t    trace_capacity;
    int32_t     order_stride; /* column stride of CHAIN_ORDER_STRIDED; 0 = 2 */
    int32_t     debug_first_skip; /* test knob, 0 or 1, as in chain_conv_args */
} chain_attn_args;

chain_status chain_attn(const void* Q, const void* K, const void* V, void* O,
                        int B, int heads, int S, int d, float scale, int policy);
chain_status chain_attn_ex(const chain_attn_args* a);
size_t chain_attn_workspace_bytes(int B, int heads, int S, int d, int policy,
                                  int dtype, int tile_cfg);

/* Self-attention block, three dependent kernels in one launch (cuSync paper,
 * Fig. "Architecture of two building blocks of GPT models" (b), section
 * "Self-Attention"): XQKV = X Wqkv (X [M,H], Wqkv [H, 3*Hs], Hs = heads*d,
 * stored fp16); per head h the fused dot product
 * XDot[:, h*d:(h+1)*d] = softmax_rows(scale * Q_h S2_h^T) S3_h over all M
 * tokens, where Q_h, S2_h, S3_h are head h's columns of the first, second and
 * third slice of XQKV (fp32 softmax, no mask or dropout, stored fp16); then
 * Y = XDot W2 (W2 [Hs,H]).  Policies: STREAM_SERIAL (three stream-ordered
 * launches), STRIDEDSYNC, TILESYNC (stage 2 checks each stage-1 tile's own
 * flag).  This build supports d = 128, any M >= 1 (a partial last row tile
 * and query block; keys past M take no probability), H a multiple of 128. */
typedef struct chain_selfattn_args {
    const void* X;            /* [M,H] */
    const void* Wqkv;         /* [H,3*heads*d] */
    const void* W2;           /* [heads*d,H] */
    void*       Y;            /* [M,H] output */
    int64_t     M, H;
    int32_t     heads, d;
    float       scale;        /* softmax scale (e.g. 1/sqrt(d)) */
    int32_t     policy;       /* STREAM_SERIAL | STRIDEDSYNC | TILESYNC */
    int32_t     dtype;        /* CHAIN_F16 or CHAIN_BF16 */
    int32_t     split_k1;     /* K splits of a stage-1 (XQKV) tile: 0 = automatic (by shape:
                                 within one wave of 256 tiles, the split that finishes in the
                                 fewest rounds of a fraction of a tile when that saves a third;
                                 past one wave, only the tiles after the last whole wave, see
                                 chain_selfattn_plan), 1 = none, s > 1: s splits of every tile
                                 (s must divide H / 64); deterministic reduction */
    void*       stream;
    void*       workspace;
    size_t      workspace_bytes;
    void*       qkv_out;      /* optional [M,3*heads*d] buffer for XQKV; NULL = workspace */
    void*       dot_out;      /* optional [M,heads*d] buffer for XDot; NULL = workspace */
    uint64_t    order_seed;
    int32_t     order;        /* CHAIN_ORDER_*: one group per stage for the table orders */
    int32_t     grid;
    uint32_t    poll_limit;
    int32_t     debug_skip_producer; /* 0 = none; k > 0: work item k-1 (stage 1 items, a
                                        tile's K splits adjacent, then stage 2 items, an
                                        item's key splits adjacent) never posts */
    uint32_t    debug_delay;
    int32_t     split_keys;   /* key splits of a stage-2 (query block, head) item: 0 =
                                 automatic (split when those items do not fill the GPU),
                                 1 = none, s > 1: s contiguous ranges of 64-key blocks, each
                                 non-empty; the last split to finish merges the partial
                                 softmax states in split order (deterministic) */
    void*       trace;        /* optional per-item trace, as in chain_mlp_args: the work items
                                 as chain_selfattn_plan counts them (stage 1, then 2, then 3) */
    uint32_t    trace_capacity;
} chain_selfattn_args;

chain_status chain_selfattn(const void* X, const void* Wqkv, const void* W2, void* Y, int64_t M,
                            int64_t H, int heads, int d, float scale, int policy);
chain_status chain_selfattn_ex(const chain_selfattn_args* a);
size_t chain_selfattn_workspace_bytes(int64_t M, int64_t H, int heads, int d, int policy,
                                      int dtype);

/* ---- workspace, status ------------------------------------------------------
 * A workspace holds the intermediate (unless z_out/s_out is given), the
 * readiness flags, the work counters, the order table and a status block.
 * It must be zeroed before first use (chain_workspace_reset) and is then
 * self-maintaining: the last workgroup of every launch resets the counters. */
chain_status chain_workspace_reset(void* workspace, size_t bytes, void* stream);
/* Synchronise the stream, then return CHAIN_ETIMEOUT (and clear it) if a
 * device wait in this workspace expired since the last check, else CHAIN_OK. */
chain_status chain_workspace_status(void* workspace, void* stream);
/* Same for the library-owned workspace of the current device. */
chain_status chain_sync(void* stream);
/* Free the library-owned workspaces of all devices. */
void chain_release(void);

const char* chain_strerror(chain_status s);
int chain_last_hip_error(void);                      /* last hipError_t seen (0 = none) */
/* Producer/consumer work item and kind (0 producer, 1 consumer) of the last
 * reported watchdog expiry; CHAIN_OK if one was recorded, CHAIN_EINVAL if not. */
chain_status chain_last_timeout(int64_t* item, int* kind);

/* ---- host-side planning helpers (no GPU needed) ----------------------------- */
typedef struct chain_tile_info {
    int32_t bm, bn1, bn2;     /* producer tile BM x BN1, consumer tile BM x BN2 */
    int32_t bk;               /* K step staged per LDS buffer */
    int32_t threads;          /* threads per workgroup */
    int32_t lds_bytes;        /* LDS per workgroup */
} chain_tile_info;

int chain_num_tile_cfgs(void);
chain_status chain_tile_cfg_info(int cfg, chain_tile_info* out);

typedef struct chain_plan {
    int32_t tile_cfg;
    int64_t row_tiles;        /* ceil(M / BM) */
    int64_t prod_col_tiles;   /* F / BN1 */
    int64_t cons_col_tiles;   /* H / BN2 */
    int64_t producer_tiles;   /* P */
    int64_t consumer_tiles;   /* C */
    int32_t split_k1;         /* K splits per producer tile (1 = none) */
    int32_t split_k2;         /* K splits per consumer tile */
} chain_plan;
/* Tile configuration and tile counts the MLP chain would use. */
chain_status chain_mlp_plan(int64_t M, int64_t H, int64_t F, int dtype, int tile_cfg,
                            chain_plan* out);
/* Tile configuration (an index of the conv tile table, pixels x channels and
 * ring stages: 0 128x64/3, 1 256x64/3, 2 128x128/3, 3 64x64/4, 4 128x64/2,
 * 5 64x64/3, 6 64x64/2, 7 128x128/2), tile counts and K splits the 3x3
 * conv pair (pad 1, stride 1, fp16) would use for N images of Hh x Ww with C
 * input and K output channels; row tiles count flattened output pixels.
 * tile_cfg < 0 = automatic.  The same checks as chain_conv_ex, no device
 * call. */
chain_status chain_conv_plan(int N, int Hh, int Ww, int C, int K, int tile_cfg, chain_plan* out);

typedef struct chain_selfattn_plan_info {
    int32_t row_tile, col_tile; /* stage 1 and 3 tiles (rows x columns) */
    int64_t row_tiles;        /* ceil(M / row_tile) */
    int64_t stage1_tiles;     /* row_tiles x 3 x heads (the three slices of every head) */
    int32_t split_k1;         /* K splits of a stage-1 tile (1 = none) */
    int32_t split_keys;       /* key splits of a stage-2 item (1 = none) */
    int64_t query_blocks;     /* ceil(M / 256): queries per stage-2 item */
    int64_t key_blocks;       /* ceil(M / 64): keys per stage-2 pipeline step */
    int64_t stage1_items;     /* (stage1_tiles - tail_tiles) x split_k1 + tail_tiles x split_k_tail */
    int64_t stage2_items;     /* query_blocks x heads x split_keys */
    int64_t stage3_items;     /* row_tiles x H / col_tile */
    int64_t tail_tiles;       /* the last stage-1 tiles in item order, split split_k_tail ways
                                 (automatic split_k1 only: the tiles past the last whole wave
                                 of 256 when the tiles fill more than one; else 0) */
    int32_t split_k_tail;     /* K splits of a tail tile (1 = none) */
    int32_t reserved;
} chain_selfattn_plan_info;
/* Tiles, splits and work items the self-attention chain would use for these
 * shapes and split requests (0 = automatic, as in chain_selfattn_args); the
 * same argument checks as chain_selfattn_ex, with no device call.  Work items
 * are numbered stage after stage (the numbering of debug_skip_producer). */
chain_status chain_selfattn_plan(int64_t M, int64_t H, int heads, int d, int split_k1,
                                 int split_keys, chain_selfattn_plan_info* out);

/* Work order of a call (no GPU needed): the work items in the order the
 * persistent workgroups take them, as the _ex call with these arguments
 * would hand them out (its plan, order, seed and stride; pointers and sizes
 * are checked as there).  One global counter: the whole sequence, producer
 * items numbered first (0 .. producer items - 1, K splits adjacent).  Per-XCD
 * queues (CHAIN_ORDER_XCD where it applies): the queue lists, phase after
 * phase; a workgroup starts consumer queues only once every producer queue is
 * empty.  *count receives the number of items; items may be NULL to ask for
 * it, else capacity must be at least that (CHAIN_EINVAL otherwise).  These
 * sequences are what the deadlock-freedom argument is about: every consumer
 * item comes after all the producer items it reads (cuSync paper, "Tile
 * Processing Order" and "Stage Processing Order"). */
chain_status chain_mlp_order(const chain_mlp_args* a, uint32_t* items, size_t capacity,
                             size_t* count);
chain_status chain_conv_order(const chain_conv_args* a, uint32_t* items, size_t capacity,
                              size_t* count);
chain_status chain_attn_order(const chain_attn_args* a, uint32_t* items, size_t capacity,
                              size_t* count);

/* Measurement calibration (not on the cuSync pages): the sustained dense fp16
 * MFMA rate and shader clock of the current device.  One launch of
 * CUs x waves_per_simd (1 or 2) workgroups of four waves; each wave runs
 * iters rounds of eight independent 32x32x16 fp16 MFMA chains on
 * pseudo-random register operands and nothing else.  scratch: caller device
 * memory of at least CUs * waves_per_simd * 1280 bytes (16-byte aligned).
 * Synchronises the stream; returns the achieved TFLOP/s, the average shader
 * clock in GHz (shader clock counter over the 100 MHz realtime counter) and
 * the launch time in ms.  The published peak assumes the top clock; under a
 * sustained MFMA load the chip's power management may run lower, and this
 * call measures what it runs at. */
chain_status chain_calibrate_mfma(int waves_per_simd, int iters, void* scratch,
                                  size_t scratch_bytes, void* stream, double* tflops,
                                  double* ghz, double* ms);

/* Measurement calibration: copies `bytes` (a multiple of 16, below 2 GiB)
 * from src to dst (device pointers, 16-byte aligned, not overlapping) with 16-
 * byte buffer loads and stores like the chain kernels', asynchronously on
 * `stream`: a kernel of known traffic (bytes read, bytes written) against
 * which hardware traffic counters are scaled. */
chain_status chain_calibrate_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Wave model of the cuSync paper, section "Thread block Wave Execution":
 * a kernel of b blocks on a GPU running `slots` blocks at once takes
 * ceil(b / slots) waves.  For n dependent kernels, frac[i] = blocks[i]/slots,
 * *serial_waves = sum ceil(blocks[i]/slots) (stream synchronisation) and
 * *fused_waves = sum(blocks)/slots (all blocks share waves). */
chain_status chain_wave_model(const int64_t* blocks, int n, int64_t slots,
                              double* frac, int64_t* serial_waves, double* fused_waves);

/* Conv2DTileSync halo range: the first and last producer pixel-tile index a
 * consumer pixel tile reads, for tiles of bm flattened output pixels of an
 * N x Hh x Ww image batch, an R x S window with padding pad, stride 1. */
chain_status chain_conv_dep_range(int64_t tile, int64_t N, int64_t Hh, int64_t Ww,
                                  int64_t bm, int R, int S, int pad,
                                  int64_t* first, int64_t* last);

#ifdef __cplusplus
}
#endif
#endif /* TLSYNC_H */
