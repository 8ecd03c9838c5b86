/*
 * atlas.h -- C ABI of libatlas: exact causal grouped-query attention over a
 * paged K/V cache on AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  For sequence b with context length L_b (keys at
 * positions 0..L_b-1) and q_len queries that are the suffix of that history
 * (query i sits at position pos = L_b - q_len + i; CPUAttn README, "Parallel
 * example", cache-backed semantics), and q-head h reading K/V head g =
 * head_map[h] (CPUAttn "Operator model": standard, GQA, MQA):
 *
 *     visible(j) = j <= pos  and  (W_b == 0  or  j > pos - W_b  or  j < S_b)
 *     s_j        = scale * <q, K_g[j]>
 *     s_j        = c_b * tanh(s_j / c_b)                 if softcap c_b > 0
 *     out        = sum_j softmax_j(s) * V_g[j]  over visible j
 *     lse        = log sum_j exp(s_j)           over visible j
 *
 * The window / sink / softcap variants are named by the ferrox-core crate
 * index (causal_gqa_attention_windowed, _sinks, _softcap, _paged_sinks,
 * _windowed_softcap); the pages give no formulas, and the readings above are
 * the ones this library implements.  The K/V history is paged: the CFR-Atlas
 * README ("Core contract") requires the page-by-page folded result to equal
 * full-K/V attention, which is what these entry points return: every visible
 * key is read, nothing is pruned or approximated; the pages are folded into
 * online-softmax states (max, sum, accumulator) and the partial states are
 * merged exactly (log-sum-exp merge; CPUAttn "Operator model", split-K only
 * with a structured merge).
 *
 * Memory layout (all row-major, all caller-owned; the library never
 * allocates device memory):
 *   q           [B][q_len][Hq][D]                 (q_dtype)
 *   k_pages     [num_phys_pages][Hkv][P][D]       (kv_dtype) one (page, head)
 *   v_pages     [num_phys_pages][Hkv][P][D]       slab is K[token][dim],
 *                                                 CFR-Atlas "Minimal integration"
 *   page_table  [B][max_pages_per_seq] int32      logical page -> physical id
 *   context_lens[B] int32                         L_b
 *   window, sink_tokens [B] int32, softcap [B] f32  optional (NULL = off)
 *   out         [B][q_len][Hq][D] f32
 *   lse         [B][q_len][Hq] f32                optional (NULL = not written)
 * Rows of a sequence's last page past L_b, and physical pages no page table
 * references, are never read, whatever they hold.
 *
 * Calls are asynchronous on the caller's HIP stream (a hipStream_t passed as
 * void*, NULL = the null stream) and never synchronise the host, except in
 * validation mode (environment ATLAS_VALIDATE=1), which copies the device
 * page table and lengths to the host and checks them before launching.
 * With the environment variable ATLAS_DEBUG set, each attention call prints
 * one line to stderr naming the kernels it chose (tiled or split-KV) and
 * their plan.
 *
 * Errors.  Every check of host-visible arguments runs before any launch: on
 * an error nothing is launched and no output is written.  The detail of the
 * last error on the calling thread is returned by atlas_last_error().
 * Device-resident values (page ids, lengths, window/sink counts) are trusted
 * outside validation mode; kernels clamp them so that no access leaves the
 * caller's buffers, and a query row with no visible key (possible only when
 * q_len > L_b) yields NaN outputs and lse = -inf.
 *
 * Thread safety: the functions keep no state between calls (only a
 * thread-local error string), so concurrent calls on different streams with
 * disjoint outputs and workspaces are safe.
 */
#ifndef ATLAS_H
#define ATLAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATLAS_ABI_VERSION 2

/* Status codes returned by every entry point.  The CFR-Atlas README
 * ("Validation and hardening") rejects invalid configuration and non-finite
 * inputs with an error instead of a partial result; the ferrox-core crate
 * index ("kernel_registry") makes a missing kernel a loud error.  These codes
 * are how this library reports both. */
enum {
    ATLAS_OK = 0,
    ATLAS_ERR_NULL = 1,        /* a required pointer is NULL */
    ATLAS_ERR_SHAPE = 2,       /* bad sizes, Hq % Hkv != 0 without head_map, bad head_map entry */
    ATLAS_ERR_RANGE = 3,       /* a size or count out of range (e.g. q_len > max context) */
    ATLAS_ERR_UNSUPPORTED = 4, /* no kernel for this dtype / head_dim / page size: never a silent fallback */
    ATLAS_ERR_WORKSPACE = 5,   /* workspace smaller than the matching *_workspace_bytes(), or not 16-byte aligned */
    ATLAS_ERR_POOL = 6,        /* validation mode: a page id outside [0, num_phys_pages) */
    ATLAS_ERR_NONFINITE = 7,   /* validation mode: a NaN or Inf in the visible inputs */
    ATLAS_ERR_DEVICE = 8       /* a HIP runtime error */
};

/* Element types of q (q_dtype) and of k_pages / v_pages (kv_dtype). */
enum {
    ATLAS_DTYPE_F32 = 0,
    ATLAS_DTYPE_BF16 = 1
};

/*
 * Arguments of one attention call.  Supported: head_dim 64 or 128; page_size
 * a power of two in [1, 4096]; Hq, Hkv <= 256; (q_dtype, kv_dtype) one of
 * (f32, f32), (bf16, bf16) or (f32, bf16) -- an fp32 query over a bf16 cache
 * -- else ATLAS_ERR_UNSUPPORTED.  The CPUAttn README ("Parallel example")
 * passes Q, K and V as separate caller-owned tensors, K/V read-only.
 */
typedef struct atlas_attn_args {
    int32_t q_dtype;            /* ATLAS_DTYPE_* of q */
    int32_t kv_dtype;           /* ATLAS_DTYPE_* of k_pages and v_pages */
    int32_t batch;              /* B >= 1 */
    int32_t q_len;              /* queries per sequence (1 for decode) */
    int32_t num_q_heads;        /* Hq */
    int32_t num_kv_heads;       /* Hkv */
    int32_t head_dim;           /* D */
    int32_t page_size;          /* P, tokens per page */
    int32_t num_phys_pages;     /* pages in each arena */
    int32_t max_pages_per_seq;  /* columns of page_table; every L_b <= max_pages_per_seq * P */
    int32_t split_tokens;       /* keys per split-KV work item; 0 = library's choice
                                   (results depend on it only through rounding order) */
    float scale;                /* score scale, finite and > 0, e.g. 1/sqrt(D) */
    const int32_t *head_map;    /* HOST [Hq] -> K/V head, or NULL for h / (Hq / Hkv) */
    const void *q;              /* device, see layout above */
    const void *k_pages;        /* device */
    const void *v_pages;        /* device */
    const int32_t *page_table;  /* device */
    const int32_t *context_lens;/* device */
    const int32_t *window;      /* device [B] or NULL; 0 = no window for that sequence */
    const int32_t *sink_tokens; /* device [B] or NULL; only used where window > 0 */
    const float *softcap;       /* device [B] or NULL; 0 = no softcap for that sequence */
    float *out;                 /* device */
    float *lse;                 /* device or NULL */
    void *workspace;            /* device scratch, >= the matching *_workspace_bytes(), 16-byte aligned */
    size_t workspace_bytes;
} atlas_attn_args;

/* One page to regenerate: page `logical_page` of the sequence whose generator
 * key is `seq` (in [0, 65536); other values make the job a no-op) is written
 * into physical page `phys_page` of both arenas (all Hkv heads). */
typedef struct atlas_regen_job {
    int32_t seq;
    int32_t logical_page;
    int32_t phys_page;
} atlas_regen_job;

/*
 * Arguments of one regeneration call.  The CFR-Atlas README ("Minimal
 * integration") has the backend replay exact row-major K[token][dim] and
 * V[token][dim] rows of one (layer, K/V head, token range) on demand; this
 * library's replay is a seeded counter-based generator: value (tensor t in
 * {1 = K, 2 = V}, head h, token j, dim d) is the Box-Muller normal built from
 * Philox4x32-10 (Salmon et al., SC'11) with key = seed and counter
 * (j, d / 4, h | t << 30, layer | seq << 16): words 0,1 give dims 4k, 4k+1
 * as r cos(2 pi u1), r sin(2 pi u1) with r = sqrt(-2 ln u0), words 2,3 give
 * dims 4k+2, 4k+3, and word x maps to u = (floor(x / 512) + 1/2) * 2^-23.
 * Computed in fp32; bf16 arenas store it rounded to nearest-even.
 * Requires layer < 2^16 and Hkv < 2^30 (ATLAS_ERR_RANGE); jobs with seq
 * outside [0, 2^16) are skipped.
 */
typedef struct atlas_regen_args {
    uint64_t seed;
    int32_t layer;
    int32_t dtype;              /* ATLAS_DTYPE_* of the arenas */
    int32_t num_kv_heads;
    int32_t head_dim;           /* 64 or 128 */
    int32_t page_size;          /* power of two in [1, 4096] */
    int32_t num_phys_pages;
    int32_t num_jobs;           /* >= 0 */
    int32_t reserved0;
    const atlas_regen_job *jobs;/* device [num_jobs]; jobs with phys_page outside
                                   [0, num_phys_pages), seq outside [0, 65536) or
                                   logical_page < 0 are skipped */
    void *k_pages;              /* device arena */
    void *v_pages;              /* device arena */
} atlas_regen_args;

/* ABI version of the loaded library (ATLAS_ABI_VERSION at build time).  The
 * CPUAttn README ("Runtime ownership") keys its compiled artifacts by ABI so
 * that a caller never runs code built against another argument layout; a
 * binding compares this value with the version it was written for. */
int32_t atlas_abi_version(void);

/* Static description of a status code (never NULL; "unknown status" for a
 * value outside the enum).  CFR-Atlas README, "Validation and hardening":
 * rejected configuration is reported, not silently repaired. */
const char *atlas_status_str(int32_t status);

/* Detail of the last non-OK status returned on the calling thread ("" after
 * a successful call or if none); the string is owned by the library and valid
 * until the thread's next call.  Same passage as atlas_status_str. */
const char *atlas_last_error(void);

/* Workspace bytes atlas_attend_decode / atlas_attend_prefill (and
 * atlas_attend_mods, atlas_attend_decode_regen) need for these arguments; only
 * the sizes are read, pointers are not inspected.  The CPUAttn README
 * ("Runtime ownership") keeps workspace and output allocation outside the
 * timed native call; here the caller allocates the workspace once (device
 * memory, any alignment of 256 bytes or more) and may reuse it for every call
 * that fits in it; its contents need no initialisation.  Returns SIZE_MAX
 * when the sizes are invalid (the reason is in atlas_last_error()). */
size_t atlas_decode_workspace_bytes(const atlas_attn_args *args);
size_t atlas_prefill_workspace_bytes(const atlas_attn_args *args);

/*
 * Decode: one query per sequence (q_len must be 1) at position L_b - 1 (the
 * CFR-Atlas README, "Minimal integration", passes the context length
 * including the current token).  The CFR-Atlas README ("Core contract") folds
 * each page into an online-softmax state and requires the folded result to
 * equal full-K/V attention; the CPUAttn README ("Operator model") allows a
 * split over keys only with a structured merge.  Here each (sequence, K/V
 * head, span of keys) work item folds its keys into an online-softmax state
 * for the q-heads of that K/V head (up to 16 of them per work item on the
 * matrix cores, 8 on the vector ALUs), and a log-sum-exp merge combines the
 * states of each (sequence, q-head) in a fixed span order (deterministic:
 * the same arguments give the same bits, whatever the physical page order).
 * Decode always runs these split-KV kernels, so that its results equal
 * those of atlas_attend_decode_regen bit for bit; a single query through
 * atlas_attend_prefill may take the tiled kernels instead (see there).
 * Arguments as described above; workspace >= atlas_decode_workspace_bytes().
 */
int32_t atlas_attend_decode(const atlas_attn_args *args, void *stream);

/*
 * Prefill / cache-backed short queries: q_len >= 1 queries per sequence, the
 * suffix of the history (requires q_len <= L_b).  A tiled call is one with
 * q and K/V of one dtype and q_len >= 64, or with q_len * G above 32 rows for a bf16 cache or above 8
 * for fp32 (G = the largest number of q-heads reading one K/V head) and
 * batch * q_len * max_pages_per_seq * page_size at least 2^17 (2^16 for
 * fp32 with q_len >= 2).  A tiled bf16 call runs
 * the tiled matrix-core kernel (query x key tiles with causal block-stop:
 * each query tile stops at the last key tile its last row can see, and with
 * a window it also skips the key tiles before its first row's window, except
 * those holding sink keys).  Its P.V product runs in fp16 with
 * fp32 accumulation, so it requires |V| <= 65504 (validation mode checks
 * this and returns ATLAS_ERR_RANGE).  A tiled fp32 call runs the same
 * tiling on the fp16 matrix cores with every operand split into two fp16
 * parts (hi = fp16(x), lo = fp16(x - hi)) and each product taken as
 * hi.hi + lo.hi + hi.lo, which keeps fp32 accuracy (CPUAttn defines the
 * method on FP32 tensors).  Q and K rows are first scaled by powers of two
 * into the fp16 range, so any finite q and k elements below 2^115 in
 * magnitude are taken (the scores scale * q.k still have to stay within the
 * fp32 softmax's range, |score| < 2^26); V is split unscaled, so this path
 * requires |v| <= 65504 (validation
 * mode: ATLAS_ERR_RANGE).  On both tiled paths a V value beyond 65504 is
 * outside the kernel's domain: validation mode rejects the call, and without
 * validation the rows that read it come out inf or NaN (the split-KV kernels
 * below take any finite V).  Every other case runs the split-KV kernels of
 * atlas_attend_decode with each (query, q-head) pair as a row.
 */
int32_t atlas_attend_prefill(const atlas_attn_args *args, void *stream);

/*
 * Score and mask modifications.  CPUAttn ("Operator model") defines Parallel
 * attention as standard (non-causal) or causal, with elementwise score and
 * mask expressions, and its tiled lowering keeps an arbitrary mask's
 * elementwise meaning ("Parallel lowerings").  Here:
 *   causal        1: key j is visible to a query at position pos only if
 *                 j <= pos (the rule of atlas_attend_prefill); 0: every key
 *                 j < L_b is visible (window and sink_tokens must be NULL,
 *                 else ATLAS_ERR_UNSUPPORTED).
 *   alibi_slopes  device [num_q_heads] fp32, or NULL: the logit of key j for
 *                 q-head h gains -alibi_slopes[h] * |pos - j|, after the
 *                 softcap and before the mask (ALiBi-style linear bias).
 *   mask_bits     device [batch][q_len][mask_words] uint32, or NULL: key j of
 *                 query row i of sequence b is visible only if bit (j & 31)
 *                 of word (j >> 5) of row (b, i) is set; ANDed with the
 *                 causal / window / sink rule.  Bits of keys >= L_b are
 *                 ignored.
 *   mask_words    words per mask row, >= ceil(max_pages_per_seq * page_size
 *                 / 32) when mask_bits is set (else ATLAS_ERR_SHAPE).
 * A row whose visible set is empty gets NaN output and lse = -inf.
 */
typedef struct atlas_attn_mods {
    int32_t causal;
    int32_t mask_words;
    const float *alibi_slopes;
    const uint32_t *mask_bits;
} atlas_attn_mods;

/*
 * atlas_attend_prefill with modifications (mods may be NULL: no
 * modification).  Same arguments, workspace (atlas_prefill_workspace_bytes)
 * and outputs; q_len >= 1.  Tiled calls (as for atlas_attend_prefill) run
 * the tiled kernels (non-causal rows take every key block of the context;
 * a mask's fully hidden key blocks are skipped, masked and biased elements
 * are applied per element inside the others); every other case runs the
 * split-KV kernels.
 */
int32_t atlas_attend_mods(const atlas_attn_args *args, const atlas_attn_mods *mods, void *stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * decode as atlas_attend_decode (same kernels, same results to the bit), but
 * the split partial states live in a device array inside the library instead
 * of a caller workspace: args->workspace and args->workspace_bytes are
 * ignored, the caller passes only inputs and outputs, and the call allocates
 * nothing (no hipMalloc, no host allocation).  The array holds
 * ATLAS_NOALLOC_SCRATCH_BYTES (32 MiB) on each GPU the library runs on, from
 * the first call on that GPU until the process ends; a decode whose partial
 * states need more (atlas_decode_workspace_bytes() above that) returns
 * ATLAS_ERR_WORKSPACE before anything runs.  Calls on the current device's
 * streams only (ATLAS_ERR_DEVICE for a stream of another device).  Every
 * call on one GPU uses the same array: calls that overlap in time on one GPU
 * (several streams, several threads) race and must be serialised by the
 * caller.  Validation mode (ATLAS_VALIDATE=1) is not available here
 * (ATLAS_ERR_UNSUPPORTED): it copies device arrays to host buffers.
 */
#define ATLAS_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int32_t atlas_attend_decode_noalloc(const atlas_attn_args *args, void *stream);

/* Regenerate whole pages (all heads, all P tokens) into the arenas. */
int32_t atlas_regenerate_pages(const atlas_regen_args *args, void *stream);

/* Page-table value of a page that is not stored (atlas_attend_decode_regen). */
#define ATLAS_PAGE_REGENERATE (-1)

/*
 * Decode with cold pages regenerated inside the attention kernel.  The
 * CFR-Atlas README ("Core contract") replays a cold page on demand and
 * requires attention over replayed pages to equal attention over stored
 * ones; here the replay happens in the kernel's registers instead of a
 * scratch page, so a cold page costs generator arithmetic but no HBM
 * traffic.  Same as atlas_attend_decode (same arguments, workspace and
 * output), except that page_table entries equal to ATLAS_PAGE_REGENERATE
 * stand for the rows atlas_regenerate_pages would write for
 * (seed, layer, key seq_keys[b], that logical page): the result equals
 * regenerating those pages into the pool and calling atlas_attend_decode, to
 * the bit.  Nothing of such a page is read from the arenas.
 *   seq_keys  device [B] int32, each sequence's generator key in [0, 65536)
 *             (a persistent sequence id, so that a sequence keeps its K/V when
 *             it moves to another batch row between calls), or NULL: the key
 *             is the batch row b.  Keys outside [0, 65536) are clamped into it
 *             outside validation mode (ATLAS_ERR_RANGE in validation mode).
 * kv_dtype f32 or bf16 (any q_dtype pairing atlas_attend_decode takes);
 * requires layer in [0, 65536) (ATLAS_ERR_RANGE).  Validation mode accepts
 * ATLAS_PAGE_REGENERATE entries.
 */
int32_t atlas_attend_decode_regen(const atlas_attn_args *args, uint64_t seed, int32_t layer,
                                  const int32_t *seq_keys, void *stream);

/*
 * Appending K/V rows: the decode step's write of each sequence's new tokens
 * into their pages (CPUAttn README, cache-backed decode streams that grow by
 * one token per step).  Token t of sequence b (t < n_new) sits at position
 * p = start_pos[b] + t and is written, for every K/V head, into row p % P of
 * physical page page_table[b][p / P] of both arenas; nothing else is
 * written.  The new rows' layout is [B][n_new][Hkv][D] in the arenas' dtype.
 * Device-resident values are trusted outside validation mode, where a target
 * page outside the pool returns ATLAS_ERR_POOL and a position outside
 * [0, max_pages_per_seq * P) returns ATLAS_ERR_RANGE before anything is
 * written; otherwise rows whose page id or position is out of range are
 * skipped (never written elsewhere).
 */
typedef struct atlas_append_args {
    int32_t dtype;              /* ATLAS_DTYPE_* of the arenas and the new rows */
    int32_t batch;              /* B >= 1 */
    int32_t n_new;              /* tokens appended per sequence, >= 0 */
    int32_t num_kv_heads;       /* Hkv */
    int32_t head_dim;           /* D, 64 or 128 */
    int32_t page_size;          /* P, power of two in [1, 4096] */
    int32_t num_phys_pages;
    int32_t max_pages_per_seq;
    const void *k_new;          /* device [B][n_new][Hkv][D] */
    const void *v_new;          /* device [B][n_new][Hkv][D] */
    const int32_t *page_table;  /* device [B][max_pages_per_seq] */
    const int32_t *start_pos;   /* device [B]: position of each sequence's first new token */
    void *k_pages;              /* device arena [num_phys_pages][Hkv][P][D] */
    void *v_pages;              /* device arena */
} atlas_append_args;

int32_t atlas_append_kv(const atlas_append_args *args, void *stream);

/*
 * Page pool: host-side bookkeeping of the physical pages of a pair of arenas
 * (the caller owns the arenas).  Pages carry reference counts so that a
 * prefix's pages can be shared by several sequences' page tables and return
 * to the pool when the last user releases them.  CFR-Atlas README ("Core
 * contract"): an exhausted pool is an error, never a silent eviction.  All
 * functions are safe to call from several threads.
 */
typedef struct atlas_pool atlas_pool;

/* A pool of num_pages (>= 1) free pages with ids 0 .. num_pages-1. */
int32_t atlas_pool_create(int32_t num_pages, atlas_pool **out);
void atlas_pool_destroy(atlas_pool *pool);

/* Take n free pages (reference count 1), lowest free ids first after a
 * fresh create; all or nothing: ATLAS_ERR_POOL when fewer than n are free. */
int32_t atlas_pool_alloc(atlas_pool *pool, int32_t n, int32_t *ids);

/* Add one reference to each listed page (each must be in use), e.g. when
 * another sequence starts sharing a prefix.  ATLAS_ERR_RANGE if any id is
 * out of range or free (then nothing changes). */
int32_t atlas_pool_retain(atlas_pool *pool, int32_t n, const int32_t *ids);

/* Drop one reference from each listed page (an id may repeat); pages whose
 * count reaches 0 become free.  ATLAS_ERR_RANGE if any id is out of range or
 * would drop below 0 (then nothing changes). */
int32_t atlas_pool_release(atlas_pool *pool, int32_t n, const int32_t *ids);

/* Number of free pages; reference count of one page (-1 if out of range). */
int32_t atlas_pool_free_pages(const atlas_pool *pool);
int32_t atlas_pool_refcount(const atlas_pool *pool, int32_t id);

/*
 * Byte-bounded hot-page cache (host side).  The CFR-Atlas README keeps
 * selected K/V pages in a byte-bounded hot cache and regenerates the rest;
 * the library owns residency, eviction and accounting, the caller picks the
 * budget (Config::hot_cache_bytes) and the admission policy
 * (admit_regenerated_pages, KeepRecent { recent_tokens }), and admission
 * changes latency and residency only, never the attention result ("Core
 * contract").
 *
 * The resident pages occupy a hot pool of physical pages 0 .. capacity - 1
 * (capacity = hot_cache_bytes / page_bytes) in the caller's arenas; pages not
 * in the pool are regenerated inside atlas_attend_decode_regen, so cold pages
 * need no scratch memory.  A page is identified by (sequence id, layer,
 * logical page).  All functions are thread-safe per cache; on an error
 * nothing changes.
 */
typedef struct atlas_cache atlas_cache;

typedef struct atlas_cache_config {
    int64_t hot_cache_bytes;    /* residency budget */
    int64_t page_bytes;         /* bytes one resident page occupies (K and V of all K/V heads) */
    int32_t page_size;          /* tokens per page */
    int32_t recent_tokens;      /* KeepRecent: pages holding any of a sequence's last recent_tokens
                                   tokens are admitted first, evicting if needed (0: off) */
    int32_t admit_regenerated;  /* 1: a call's other non-resident pages take the free slots */
    int32_t reserved;           /* 0 */
} atlas_cache_config;

typedef struct atlas_cache_stats {
    int64_t capacity_pages;
    int64_t resident_pages;
    int64_t resident_bytes;
    int64_t hits;               /* resident pages read, summed over calls */
    int64_t misses;             /* pages left to in-kernel regeneration, summed over calls */
    int64_t admitted;           /* pages admitted (each one regeneration job) */
    int64_t evicted;
} atlas_cache_stats;

/* Create / destroy.  ATLAS_ERR_SHAPE for non-positive sizes, ATLAS_ERR_RANGE
 * for a capacity above 2^24 pages or admit_regenerated outside {0, 1}. */
int32_t atlas_cache_create(const atlas_cache_config *config, atlas_cache **out);
void atlas_cache_destroy(atlas_cache *cache);

/*
 * Plan one attention call of `layer` over `batch` sequences (host arrays):
 * seq_ids [batch] (distinct, each in [0, 65536): a sequence id is also its
 * generator key, the seq_keys entry atlas_attend_decode_regen must be given
 * for that sequence's batch row), context_lens [batch] in [1,
 * max_pages_per_seq * page_size].  In order: the call's resident pages are hits; with
 * recent_tokens, each sequence's recent pages that are not resident are
 * admitted, newest first, into a free slot or in place of the least recently
 * used page this call does not read (pages outside every recent window
 * before those inside one; O(capacity) per eviction); with
 * admit_regenerated, the call's other non-resident pages take the slots
 * still free, in (sequence, page) order.  Writes page_table [batch]
 * [max_pages_per_seq] (host): each page's slot, or ATLAS_PAGE_REGENERATE for
 * pages left cold and for entries past the context; and admit_jobs
 * [*n_jobs][3] = (sequence id, logical page, slot) for atlas_regenerate_pages,
 * which must run before the attention call reads the admitted slots.  A
 * sequence may occupy a different batch row in every call: its resident pages
 * and its regenerated ones come from the same key.
 * max_jobs must be >= min(pages in the call, capacity) (ATLAS_ERR_SHAPE).
 * n_cold (may be NULL) receives the number of the call's pages left to
 * in-kernel regeneration; when it is 0 every page is resident, and
 * atlas_attend_decode over this page table returns the same bits as
 * atlas_attend_decode_regen without running the generator instances (their
 * placeholder loads and ordinary caching included).
 */
int32_t atlas_cache_plan(atlas_cache *cache, int32_t layer, int32_t batch, const int64_t *seq_ids,
                         const int32_t *context_lens, int32_t max_pages_per_seq, int32_t *page_table,
                         int32_t *admit_jobs, int32_t max_jobs, int32_t *n_jobs, int32_t *n_cold);

/* Free every resident page of a sequence (all layers), e.g. when it ends. */
int32_t atlas_cache_drop_sequence(atlas_cache *cache, int64_t seq_id);

/* Residency and counters. */
int32_t atlas_cache_get_stats(atlas_cache *cache, atlas_cache_stats *out);

#ifdef __cplusplus
}
#endif

#endif /* ATLAS_H */
