/*
 * fa.h -- tiled exact attention (FlashAttention forward and backward) for
 * AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation is exact attention per (batch b, head h):
 *     S = scale * Q K^T,   P = softmax over keys of S with invalid scores at -inf,
 *     O = (P o Z * s) V,   Z the keep bits, s the keep scale (below)
 * computed tile by tile with an online softmax so that no N x N matrix ever
 * reaches device memory (FlashAttention summary, xyznot.com/vi/paper/2205.14135,
 * "Method": block scores S_ij, block statistics, merged (m, l), rescaled O_i;
 * Self-Attention tutorial, infra-guide, sections 12.2-12.3 tiling and online
 * softmax).  The backward pass recomputes S and P tile by tile from the saved
 * log-sum-exp instead of storing P (summary, core ideas, recomputation;
 * azimuth.plus explainer, "three ideas in one kernel", recomputation).
 *
 * Valid pair (i, j): (causal == 0 || j <= i) && j < key_len[b] &&
 * block_mask[i / 128][j / 128] != 0.  Masks compose by AND (causal mask:
 * tutorial section 10.2, lower triangle kept including the diagonal; block
 * mask: summary, "Block-Sparse FlashAttention").  Tiles without a valid pair
 * are skipped entirely: not loaded, not computed.
 *
 * Dropout (kernel-fused, after softmax and before the product with V;
 * explainer, kernel fusion) uses Philox4x32-10 (Salmon et al., SC'11), one
 * call per block of 4 keys x 2 query rows:
 *     counter = (j >> 2, i >> 1, b*H + h, (uint32) rng_offset),
 *     key     = ((uint32) seed, (uint32)(seed >> 32)),
 * element (i, j) reads 32-bit word (j & 3), its low 16 bits u for even i and
 * its high 16 bits for odd i, and is kept iff u >= thr = min(floor(p * 2^16),
 * 2^16 - 1) with p taken as float.  For p > 0 kept entries are scaled by
 * 2^16 / (2^16 - thr), the inverse of the exact keep probability, so that
 * the expected dropped O equals the undropped one (inverted dropout).  The
 * softmax statistics (and LSE) use the undropped P.
 *
 * Conventions for every entry point:
 *  - Pointers are device memory owned by the caller (allocated by whatever
 *    allocator the caller uses), workspaces included.  The library never
 *    allocates or frees device memory and never synchronises; all work is
 *    enqueued on `stream` in order and the call returns before it completes.
 *    A workspace must not be used by two calls whose work overlaps.
 *  - Q, K, V, O, dO, dQ, dK, dV are contiguous [B][H][N][d] row-major with
 *    16-byte aligned base addresses; K, V, dK, dV have opts->kv_heads heads
 *    instead of H when that is set (grouped-query attention).  LSE and D are float [B][H][N].
 *    Outputs must not alias inputs.
 *  - LSE_i = ln sum_j exp(S_ij) over valid j (natural log, scaled scores);
 *    a row without any valid key has O = 0, LSE = -inf and zero gradients.
 *  - Validation is done on the host before any launch; on error nothing is
 *    enqueued and nothing is written.  A failed launch returns FA_ERR_HIP
 *    and fa_last_hip_error() names it.  Device-side faults are asynchronous
 *    and surface at the caller's next synchronisation.  Device-resident
 *    arguments (key_lens, block_mask) are not read on the host; key lengths
 *    are clamped to [0, N] on the device.
 *  - Supported: d in {64, 128}; dtype fp32, fp16, bf16; any N >= 1;
 *    1 <= B, H <= 65535 with N*d < 2^31 and B*H*N < 2^31; 0 <= p < 1;
 *    scale finite and > 0.
 *  - Entry points are thread-safe and keep no state between calls apart from
 *    a thread-local error string.  They only launch kernels (and record the
 *    optional timing events) on `stream`, so a call may be captured in a HIP
 *    graph and replayed; the replays read the buffers' current contents.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 7

/* FA_DTYPE_RANGE_ only widens the enum's range to 32 bits, so that any value
 * a caller passes can be read (and rejected with FA_ERR_DTYPE) without
 * undefined behaviour in the C++ implementation; it is not a dtype. */
typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2, FA_DTYPE_RANGE_ = 0x7fffffff } fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = -1,       /* a required pointer is NULL                          */
    FA_ERR_SHAPE = -2,      /* B, H or N < 1, or the tensor is too large           */
    FA_ERR_HEAD_DIM = -3,   /* d not in {64, 128}                                   */
    FA_ERR_DTYPE = -4,      /* unknown dtype                                        */
    FA_ERR_DROPOUT = -5,    /* p not in [0, 1) or not finite                        */
    FA_ERR_SCALE = -6,      /* scale not finite or <= 0                             */
    FA_ERR_ALIGN = -7,      /* a tensor base address is not 16-byte aligned         */
    FA_ERR_WORKSPACE = -8,  /* workspace NULL, too small or misaligned              */
    FA_ERR_HIP = -9,        /* a HIP launch failed (see fa_last_hip_error)          */
    FA_ERR_OPTS = -10,      /* opts->struct_size unknown or flags invalid           */
    FA_ERR_SCRATCH = -11    /* fa_bwd_noalloc: D needs more than FA_BWD_SCRATCH_BYTES */
} fa_status;

enum {
    FA_FLAG_RECORD_TILES = 1u << 0,  /* write the tile-visit map to opts->tile_visits */
    FA_FLAG_REVERSE_KV = 1u << 1     /* forward only: walk key tiles last-to-first
                                        (a check that the result does not depend on
                                        the order of the online-softmax merges)   */
};

/* Optional settings; pass NULL for all defaults.  struct_size must be
 * sizeof(fa_opts) of the caller's header (ABI versioning). */
typedef struct {
    uint32_t struct_size;
    int32_t o_fp32;             /* nonzero: O is stored as fp32 (fwd writes it, bwd
                                   reads it); 0 (and opts == NULL): O has the
                                   input dtype                                   */
    const int32_t* key_lens;    /* device int32[B]: keys j >= key_lens[b] are masked;
                                   NULL = no key padding                          */
    uint64_t rng_offset;        /* Philox counter word 3 (low 32 bits used)      */
    uint32_t flags;             /* FA_FLAG_*                                      */
    uint8_t* tile_visits;       /* device uint8[B][H][ceil(N/Br)][ceil(N/Bc)] with
                                   (Br, Bc) = fa_tile_shape(pass 0, N, causal) for
                                   fa_fwd and fa_tile_shape(pass 1, N, causal)
                                   (the dK/dV kernel as launched for this N and
                                   mask) for fa_bwd; every entry is written
                                   (1 = tile visited) when FA_FLAG_RECORD_TILES
                                   is set.  Recording does not change which
                                   kernel runs.                                  */
    uint8_t* tile_visits2;      /* fa_bwd only: the dQ kernel's map, shape from
                                   fa_tile_shape(pass 2, N, causal); may be NULL */
    hipEvent_t main_begin;      /* profiling: when both are non-NULL they are    */
    hipEvent_t main_end;        /* recorded on `stream` right before and right
                                   after the pass's main kernels (the forward
                                   kernel, without the bf16 V pre-pass; the
                                   backward's two S/P-recomputing
                                   kernels, without the D pre-pass)             */
    hipEvent_t main_mid;        /* fa_bwd profiling, optional: recorded between
                                   the dK/dV kernel and the dQ kernel            */
    int32_t kv_heads;           /* grouped-query attention: K and V (and dK, dV)
                                   are [B][kv_heads][N][d] and query head h uses
                                   K/V head h / (H / kv_heads); kv_heads must
                                   divide H (else FA_ERR_OPTS); 1 = multi-query;
                                   0 = H.  Callers whose struct_size predates
                                   this field get H.  dK, dV are summed over
                                   the query heads that share a K/V head.      */
} fa_opts;

/* Bytes of device workspace fa_fwd needs.  bf16: the forward multiplies P
 * (rounded to fp16, whose significand is 3 bits longer than bf16's) with an
 * fp16 copy of V * 2^-e_bh per (b, K/V head h): e_bh = 0 while the head's
 * largest finite |V| lies in [2^-6, 2^15), else the power of two that brings
 * it into [2^14, 2^15); every bf16 value of magnitude >= 2^(e_bh - 17)
 * converts exactly.  The workspace holds that copy (B*Hkv*N*d fp16) plus
 * 4-byte per-head statistics, each part rounded up to 256 bytes.  Hkv is
 * the number of K/V heads (opts->kv_heads, or H without grouped-query
 * attention); the value for the query head count H >= Hkv is an upper
 * bound.  fp16 and fp32 need none: 0.  Returns 0 for invalid sizes or
 * dtypes. */
size_t fa_fwd_workspace_bytes(int32_t B, int32_t Hkv, int32_t N, int32_t d, fa_dtype dtype);

/* Forward pass.  Q, K, V: [B][H][N][d] of `dtype`.  O: [B][H][N][d] of
 * `dtype`, or fp32 when opts->o_fp32 is set.  LSE: float [B][H][N].
 * causal: nonzero for the lower-triangular mask.  dropout_p in [0, 1); seed
 * selects the Philox key.  block_mask: device uint8[ceil(N/128)][ceil(N/128)],
 * shared by all (b, h), nonzero = compute; NULL = dense.  workspace: device
 * memory of at least fa_fwd_workspace_bytes(B, Hkv, N, d, dtype) bytes
 * (Hkv: the K/V heads), 256-byte aligned (may be NULL when that is 0); its
 * contents on return are unspecified. */
fa_status fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int32_t B, int32_t H, int32_t N, int32_t d, fa_dtype dtype,
                 float scale, int32_t causal, float dropout_p, uint64_t seed,
                 const uint8_t* block_mask, const fa_opts* opts,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace fa_bwd needs: D = rowsum(dO o O) as float
 * [B][H][N], rounded up to 256 bytes.  Returns 0 for invalid sizes. */
size_t fa_bwd_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d);

/* Backward pass.  Q, K, V, dO: [B][H][N][d] of `dtype`; O as the forward
 * wrote it (fp32 if opts->o_fp32, else `dtype`); LSE from the forward.  dQ, dK, dV:
 * [B][H][N][d] of `dtype`.  All of scale, causal, dropout_p, seed,
 * block_mask, key_lens and rng_offset must equal the forward call's; a
 * mismatch gives wrong gradients and is not detected.  workspace: device
 * memory of at least fa_bwd_workspace_bytes(B, H, N, d) bytes, 256-byte
 * aligned; its contents on return are unspecified.  Gradients of rows and
 * keys that take part in no valid pair are zero. */
fa_status fa_bwd(const void* Q, const void* K, const void* V, const void* O,
                 const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                 int32_t B, int32_t H, int32_t N, int32_t d, fa_dtype dtype,
                 float scale, int32_t causal, float dropout_p, uint64_t seed,
                 const uint8_t* block_mask, const fa_opts* opts,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops, harnesses that forbid allocation): fa_bwd with the
 * same arguments and contract but no workspace argument.  The D vector
 * (4 bytes per query row, B*H*N rows) lives in a static device array of
 * FA_BWD_SCRATCH_BYTES that the library holds on each GPU it runs on until
 * the process ends, so B*H*N may be at most FA_BWD_SCRATCH_BYTES / 4
 * (4,194,304 rows), else FA_ERR_SCRATCH is returned before anything is
 * enqueued.  The call allocates nothing: it looks the array's device address
 * up once per device (FA_ERR_HIP if that fails) and launches fa_bwd's
 * kernels.  Every call on one GPU shares that GPU's array: two calls whose
 * work overlaps on one GPU (on different streams, or from different threads
 * without ordering) race and may give wrong gradients; calls ordered on one
 * stream are safe.  Each call writes all of D before reading it.  The array
 * used is the one on the calling thread's current device, so `stream` must
 * belong to that device (as for fa_bwd, whose workspace must live there). */
#define FA_BWD_SCRATCH_BYTES ((size_t)16 << 20)
fa_status fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                         int32_t B, int32_t H, int32_t N, int32_t d, fa_dtype dtype,
                         float scale, int32_t causal, float dropout_p, uint64_t seed,
                         const uint8_t* block_mask, const fa_opts* opts, hipStream_t stream);

/* Decode attention over a key/value cache (Self-Attention tutorial, section
 * 11.2: the decode phase, one new token -- or a few -- per step against the
 * whole cache).  Q: [B][H][Nq][d]; K, V: [B][Hkv][Nk][d], a cache of which
 * the first kv_lens[b] rows are valid (device int32[B], clamped to [0, Nk];
 * NULL = Nk); Hkv divides H and query head h reads K/V head h / (H / Hkv).
 * Query row i of sequence b stands for position kv_lens[b] - Nq + i; with
 * `causal` it sees keys j <= that position, else all valid keys.  O:
 * [B][H][Nq][d] of `dtype`; LSE: float [B][H][Nq] (natural log, scaled
 * scores; -inf and O = 0 for a row without valid keys).  dtype: FA_BF16 or
 * FA_F16.  No dropout, no block mask, no backward.  Supported: d in {64, 128},
 * (H / Hkv) * Nq <= 65535, Nk * d < 2^31.  The cache is cut into chunks read
 * by separate workgroups whose softmax partials are merged (the two-block
 * rule of the summary's incremental softmax); workspace: device memory of at
 * least fa_decode_workspace_bytes(...) bytes, 256-byte aligned, holding those
 * partials.  events: NULL, or three events recorded on `stream` before the
 * chunk kernel, between it and the merge kernel, and after the merge (for
 * timing; the caller creates and owns them). */
size_t fa_decode_workspace_bytes(int32_t B, int32_t H, int32_t Hkv, int32_t Nq, int32_t Nk, int32_t d);
fa_status fa_decode(const void* Q, const void* K, const void* V, void* O, float* LSE,
                    int32_t B, int32_t H, int32_t Hkv, int32_t Nq, int32_t Nk, int32_t d,
                    fa_dtype dtype, float scale, int32_t causal, const int32_t* kv_lens,
                    const hipEvent_t* events, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Forward pass in the key/value-outer loop order of the original algorithm
 * (FlashAttention explainer, step-by-step algorithm; summary, "Method"):
 * for each key/value tile of block_cols keys, every query block that sees it
 * loads its running O, m, l from the workspace, updates them and stores them
 * back; the last tile a row sees writes O and LSE.  Same O and LSE as fa_fwd
 * (to rounding); kept as an IO ablation: its HBM traffic grows as
 * T_c * N * d per head (summary, "complexity": Theta(N^2 d^2 / M)), where
 * fa_fwd moves about N * d.  Q, K, V, O: [B][H][N][d] of `dtype` (FA_BF16 or
 * FA_F16); LSE float [B][H][N]; causal or not; no dropout, key padding,
 * block mask or grouped heads.  block_cols: 64 or 128 (else FA_ERR_OPTS).
 * groups_per_head: workgroups per head, each taking every G-th 128-row
 * query block (K and V are read G times per head); 0 picks
 * min(ceil(N / 128), ceil(1024 / (B*H))); more than ceil(N / 128) is
 * FA_ERR_SHAPE.  workspace: at least fa_fwd_kv_outer_workspace_bytes(...)
 * bytes, 256-byte aligned (running O fp32 [B][H][N][d], then (m, l) float
 * [B][H][N][2]).  events: NULL or two events recorded on `stream` before and
 * after the kernel. */
size_t fa_fwd_kv_outer_workspace_bytes(int32_t B, int32_t H, int32_t N, int32_t d);
fa_status fa_fwd_kv_outer(const void* Q, const void* K, const void* V, void* O, float* LSE,
                          int32_t B, int32_t H, int32_t N, int32_t d, fa_dtype dtype,
                          float scale, int32_t causal, int32_t block_cols,
                          int32_t groups_per_head, const hipEvent_t* events,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Dropout keep bits of every element, for tests: keep is device
 * uint8[B][H][N][N], 1 = kept.  Uses the same device generator as the
 * attention kernels.  O(N^2) memory: test sizes only. */
fa_status fa_dropout_keep_mask(uint64_t seed, uint64_t rng_offset, float dropout_p,
                               int32_t B, int32_t H, int32_t N, uint8_t* keep,
                               hipStream_t stream);

/* Tile shape (rows Br of queries, columns Bc of keys) of the kernel that
 * fa_fwd (pass 0) or fa_bwd (pass 1: the dK/dV kernel; pass 2: the dQ kernel)
 * launches for head dim d, dtype, sequence length N and the causal flag;
 * these index the tile-visit maps.  The dK/dV kernel has two configurations
 * (64 keys x 32 query rows for 16-bit inputs at d = 64 and for causal
 * d = 128 up to N = 2048; else 128 keys x 64 rows, fp32 x 32 rows), so its
 * shape depends on N and causal.  Both divide 128, so a tile lies inside one
 * block of the 128 x 128 block mask (summary, "Block-Sparse
 * FlashAttention": a tile is skipped iff it holds no valid pair).  Errors:
 * FA_ERR_NULL, FA_ERR_HEAD_DIM, FA_ERR_DTYPE, FA_ERR_SHAPE (N < 1),
 * FA_ERR_OPTS (unknown pass). */
fa_status fa_tile_shape(int32_t d, fa_dtype dtype, int32_t pass, int32_t N, int32_t causal, int32_t* Br,
                        int32_t* Bc);

/* Static description of a status code. */
const char* fa_status_string(fa_status s);

/* Thread-local text of the last HIP error behind FA_ERR_HIP ("" if none). */
const char* fa_last_hip_error(void);

int32_t fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
