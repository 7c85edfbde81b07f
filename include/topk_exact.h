/* topk_exact.h -- C ABI of the MI355X (gfx950) sample-guided exact Top-K selector.
 *
 * Pages cited (by title):
 *   [Cx] "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K" (codexqa.cn
 *        write-up of the HPC-Ops Top-K paper)
 *   [PD] "腾讯|长上下文稀疏注意力前K精确选择:20种配置平均加速1.55倍" (PaperDaily
 *        explainer of the same paper)
 *   [AX] "Sample-Guided Exact Top-K Selection for Long-Context Sparse Attention"
 *        (arxivdaily abstract page)
 *
 * The operation ([Cx] section "什么叫精确，时间怎么量"; [AX] abstract): for every
 * row r of an M x N_alloc FP32 score matrix whose valid prefix has length
 * L_r = row_len[r], return the indices of the K largest scores of that prefix.
 * Indices are distinct and lie in [0, L_r). When L_r > K exactly K indices are
 * returned and min(selected) >= max(unselected); boundary ties may go either way
 * and the order is unspecified. When L_r <= K all L_r valid indices are returned
 * and the remaining slots hold the caller's sentinel. There is no float
 * tolerance: scores are compared as IEEE-754 totalOrder on their 32-bit
 * patterns (so -0 < +0), which is this library's reading of "exact" on the
 * original FP32 values ([PD] question 2, Fig. 4 stage-3 caption).
 *
 * How ([PD] question 2, Fig. 4; [AX] abstract): a fixed-stride sample of the
 * row (stride 128) proposes a primary threshold tau0 aimed at about 1.5K
 * candidates and a nested, wider tau1 aimed at about 1.75K ([Cx] section
 * "采样不是处处都该开"); one mandatory full-row pass certifies the candidate
 * count, compacts the admitted candidates into LDS and builds the first radix
 * histogram; exact radix refinement then runs only on the unresolved boundary
 * bin. Underfilled or overflowing proposals fall back to exact full-row
 * recovery before anything is written. Short rows take a direct exact path.
 * All work is enqueued on the caller's stream and is graph-capturable.
 *
 * Threading and streams: the library keeps one small workspace per device
 * (control counters and statistics). Calls that overlap in time on one device
 * (for example on two streams without ordering between them) share it and race;
 * order such calls on one stream. Every pointer argument named "device" must be
 * memory of the current HIP device.
 */
#ifndef TOPK_EXACT_H
#define TOPK_EXACT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TOPK_OK = 0,
  TOPK_ERR_NULL_POINTER = 1, /* scores, row_len or out_idx is NULL while M > 0 */
  TOPK_ERR_BAD_SHAPE = 2,    /* M < 0, N_alloc < 1, N_alloc > INT32_MAX, or M*N_alloc, M*K overflow */
  TOPK_ERR_BAD_K = 3,        /* K < 1 or K > TOPK_K_MAX */
  TOPK_ERR_BAD_SENTINEL = 4, /* 0 <= sentinel < N_alloc: it would look like a valid index */
  TOPK_ERR_WORKSPACE = 5,    /* workspace missing or too small while the stream is capturing */
  TOPK_ERR_HIP = 6,          /* a HIP call or launch failed; see topk_exact_last_error() */
  TOPK_ERR_BAD_ARG = 7       /* another argument is out of range (stats/override calls) */
} topk_status_t;

#define TOPK_K_MAX 4096

/* Path override modes (test and benchmark use; default TOPK_PATH_AUTO). */
#define TOPK_PATH_AUTO 0      /* per-row choice: sentinel, direct-exact or sampled */
#define TOPK_PATH_SAMPLED 1   /* every row with L > K takes the sampled path (with line-granular
                                 sampling wherever its geometry applies) */
#define TOPK_PATH_ROWSPLIT 2  /* every row with L > K takes the sampled path, split over
                                 several workgroups (calls of at most 1024 rows) */
#define TOPK_PATH_DIRECT 3    /* every row with L > K takes the direct exact path */
#define TOPK_PATH_RECOVERY 4  /* every row with L > K takes exact full-row recovery */

/* Execution modes: how rows map to workgroups (default TOPK_EXEC_AUTO). */
#define TOPK_EXEC_AUTO 0        /* shape-based choice below */
#define TOPK_EXEC_PERSISTENT 1  /* resident workgroups loop over rows via a device ticket */
#define TOPK_EXEC_ROW_PER_WG 2  /* one workgroup per row, balanced by the hardware dispatcher */
#define TOPK_EXEC_ROWSPLIT 3    /* several workgroups per row (calls of at most 1024 rows) */

/* Statistics slots returned by topk_exact_get_stats (row counts since the last reset). */
enum {
  TOPK_STAT_ROWS = 0,            /* rows processed */
  TOPK_STAT_SENTINEL = 1,        /* rows with L <= K */
  TOPK_STAT_DIRECT = 2,          /* rows finished by the direct exact path */
  TOPK_STAT_SAMPLED = 3,         /* rows that took the sampled proposal */
  TOPK_STAT_TAU0 = 4,            /* sampled rows certified at tau0: C(tau0) >= K */
  TOPK_STAT_TAU1 = 5,            /* sampled rows with C(tau0) < K <= C(tau1) (nested fallback) */
  TOPK_STAT_RECOVER_UNDER = 6,   /* sampled rows whose admitted keys fall short of K (C(tau1) < K,
                                    or C(tau_a) < K where the deeper admission applies): exact
                                    recovery */
  TOPK_STAT_RECOVER_OVER = 7,    /* sampled rows whose candidates overflowed: exact recovery */
  TOPK_STAT_ROWSPLIT = 8,        /* rows scanned by several workgroups (row-split) */
  TOPK_STAT_FORCED_RECOVERY = 9, /* rows sent to exact recovery by TOPK_PATH_RECOVERY */
  TOPK_STAT_LONG_EXACT = 10,     /* rows longer than 16384 sample strides: sampled at a coarser
                                    fixed stride (a multiple of the set one) */
  TOPK_STAT_FRONTIER_WIDE = 11,  /* refinements whose boundary bin exceeded the frontier buffer */
  TOPK_STAT_QUEUED = 12,         /* recovery rows handed to the cooperative recovery kernels */
  TOPK_STAT_PERSISTENT = 13,     /* rows taken from the device ticket by the persistent grid */
  TOPK_STAT_ROW_PER_WG = 14,     /* rows given a workgroup of their own */
  TOPK_STAT_RECOVER_INPLACE = 15, /* recovery rows recovered by their own workgroup (rows up to
                                     262144 long, or past the cooperative queue's capacity) */
  TOPK_STAT_INPLACE_CERTIFIED = 16, /* of those: one more pass at a deeper threshold certified */
  TOPK_STAT_INPLACE_FULL = 17,   /* of those: the exact full-row select over the row ran */
  TOPK_STAT_TAUA = 18,           /* element-sampled rows with C(tau1) < K <= C(tau_a): certified
                                    at the deeper admission rank (see topk_exact_set_admission),
                                    without a second read of the row */
  TOPK_STAT_COUNT = 24
};

/* Selects the top-K indices of every row: the operation and contract of [Cx] section
 * "什么叫精确，时间怎么量" (exact set, sentinel padding of short rows, no tolerance),
 * computed by the sample-guided method of [PD] question 2 (Fig. 4) and [AX] (abstract).
 *   scores   device, row-major [M][N_alloc] float32, row stride N_alloc; read-only. Only
 *            the first clamp(row_len[r], 0, N_alloc) entries of row r are ever read.
 *   row_len  device, [M] int32, valid prefix length per row. Values outside [0, N_alloc]
 *            violate the precondition; they are clamped into it so that no access goes
 *            out of bounds, and the result for that row is then only guaranteed in-bounds.
 *   M, N_alloc, K  sizes: M >= 0, 1 <= N_alloc <= INT32_MAX, 1 <= K <= TOPK_K_MAX.
 *   out_idx  device, row-major [M][K] int32; every slot is written. For L > K: K distinct
 *            indices in [0, L), any order. For L <= K: slots [0, L) hold 0..L-1 in some
 *            order and slots [L, K) hold `sentinel`.
 *   sentinel value for empty slots; must lie outside [0, N_alloc) (e.g. -1).
 *   stream   every launch is enqueued here; the call never synchronizes, allocates or
 *            reads device memory from the host once the workspace exists (made by
 *            topk_exact_reserve or the first call outside capture), so it may be captured
 *            into a HIP graph (call topk_exact_reserve first in that case).
 * Returns TOPK_OK or an error code. Every argument and workspace error is returned before
 * anything is enqueued. TOPK_ERR_HIP from a failed launch or timing-event record may come
 * after kernels were enqueued; the call then still enqueues its recovery kernels, which
 * keep the device-side queue consistent for later calls. M == 0 is a no-op.
 * Asynchronous device faults surface on the stream like any kernel's. */
int topk_exact(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc,
               int32_t K, int32_t* out_idx, int32_t sentinel, hipStream_t stream);

/* Allocation-free variant of topk_exact, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, contract, errors and stream behaviour as topk_exact; it never calls
 * hipMalloc, hipFree or any allocating routine, needs no topk_exact_reserve, and may be
 * the first call of a process even under capture. Instead of the workspace it uses a
 * fixed scratch array in device memory of about 13.6 MB (under 16 MiB) per GPU, held
 * from library load to process end: a control block, 64 cooperative-recovery slots and
 * row-split state for 64 rows. The scratch does not grow with the call, so no call size
 * is rejected for it: calls of at most 64 rows may be row-split (larger ones run unsplit,
 * the same result), and rows needing exact recovery past the 64 queued per call are
 * recovered in place by their own workgroup. The array starts zeroed and every call
 * leaves its counters rewound for the next one. Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (different streams, or threads, without
 * ordering) race and must be serialized by the caller; it is separate from the
 * workspace topk_exact uses, so the two entry points do not race with each other.
 * Its row counters are not those topk_exact_get_stats reads, and it ignores the timing
 * hook. */
int topk_exact_noalloc(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc,
                       int32_t K, int32_t* out_idx, int32_t sentinel, hipStream_t stream);

/* Sorted, value-returning variant (an option beyond the pages' unordered contract): the
 * same selection as topk_exact, then each row's entries ordered by score descending
 * (IEEE totalOrder), ties by index ascending. For L > K: the K selected indices in that
 * order; for L <= K: all L valid indices in that order, then the sentinel.
 *   out_val  device, row-major [M][K] float32, or NULL for indices only; it receives the
 *            score of each listed index (bit for bit) and -inf in sentinel slots.
 * Other arguments, errors and capture behaviour as for topk_exact. The selected set is
 * the same as topk_exact's; which of several boundary-tied scores are kept is free, the
 * order of the output is fully determined by that set. */
/* Sorted, value-returning output (an option beside the pages' unordered contract of
 * [Cx] section "什么叫精确，时间怎么量"): the same selection as topk_exact, then each row's
 * slots ordered by score, descending in IEEE totalOrder with boundary ties by index
 * ascending; a row with L <= K lists its L indices in that order, then the sentinel.
 *   out_idx  as for topk_exact, in that order.
 *   out_val  device, row-major [M][K] float32, 4-byte aligned, or NULL: the selected scores
 *            (the input's bit patterns) in the order of out_idx, -inf in sentinel slots.
 *            With NULL only the ordered indices are written. Caller-owned.
 * Where a call has at most one row per resident workgroup and no row can be handed to the
 * recovery kernels, and in persistent calls, each row is sorted by the workgroup that
 * completes it (a selector workgroup, or the recovery finish kernel's for rows handed to
 * it); otherwise a sort kernel follows on the same stream. Capture, workspace and error behaviour as for topk_exact,
 * plus TOPK_ERR_BAD_ARG (nothing enqueued) for an out_val that is not 4-byte aligned. */
int topk_exact_sorted(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc,
                      int32_t K, int32_t* out_idx, float* out_val, int32_t sentinel, hipStream_t stream);

/* Creates the current device's workspace (control block, recovery queue and row-split
 * state, about 160 MB, one allocation) and resolves launch parameters, so that the calls
 * that follow allocate nothing. The first topk_exact call outside capture does the same;
 * the pages time only graph replays of calls whose set-up is done ([Cx] section
 * "什么叫精确，时间怎么量"), and this is that set-up. The arguments are checked (M_max >= 0,
 * 1 <= N_alloc_max <= INT32_MAX, 1 <= K <= TOPK_K_MAX) but the workspace does not depend
 * on them. Synchronous (allocates, clears and synchronizes the device); call it outside
 * stream capture before capturing topk_exact. Returns TOPK_OK, TOPK_ERR_BAD_SHAPE,
 * TOPK_ERR_BAD_K or TOPK_ERR_HIP. */
int topk_exact_reserve(int64_t M_max, int64_t N_alloc_max, int32_t K);

/* Copies up to n (<= TOPK_STAT_COUNT) statistics counters of the current device into
 * host_counts (host memory): row counts per path since the last reset. They are the
 * path rates the pages report for the proposal (rows certified at tau0, resolved by the
 * nested tau1, sent to exact recovery; [Cx] section "采样不是处处都该开"). Synchronizes
 * `stream` first. Not capturable (TOPK_ERR_BAD_ARG under capture). */
int topk_exact_get_stats(uint64_t* host_counts, int n, hipStream_t stream);

/* Zeroes the current device's statistics counters (the path rates above), enqueued on
 * `stream` as a small kernel (capturable once the workspace exists). */
int topk_exact_reset_stats(hipStream_t stream);

/* Forces one execution path for later calls (TOPK_PATH_*): the pages' boundary swap of
 * the sampled proposal against an exact one ([Cx] section "采样不是处处都该开") and the
 * forcing of every path for tests. A captured graph keeps the mode that was set when it
 * was captured. Process-wide. TOPK_ERR_BAD_ARG for an unknown mode. */
int topk_exact_set_path_override(int mode);

/* Selects how rows map to workgroups for later calls (TOPK_EXEC_*): the persistent,
 * row-split (KV-split) and one-row-per-unit executions of [AX] (abstract) and [PD]
 * (question 2). Auto uses row-split when N_alloc >= 65536 and M is at most a quarter
 * (N_alloc >= 262144) or an eighth (shorter rows) of the resident workgroup count,
 * persistent execution when M is at least four times the resident workgroup count
 * and N_alloc >= 262144, and one workgroup per row otherwise. Every mode gives a
 * result satisfying the same contract; a captured graph keeps the mode set when it
 * was captured. Row-split serves calls of at most 1024 rows. Process-wide.
 * TOPK_ERR_BAD_ARG for an unknown mode. */
int topk_exact_set_execution(int mode);

/* Proposal parameters for later calls (ablations of the pages' mechanism tables,
 * [Cx] section "采样不是处处都该开"): the sample stride s (sample keys x[j*s], j <
 * ceil(L/s)) and the primary / secondary candidate targets rho0*K and rho1*K, given
 * in thousandths of K. The method's values are s = 128, rho0 = 1.5, rho1 = 1.75
 * (restored by passing 0, 0, 0). Every setting gives an exact result; only the work
 * changes. Strides other than 128 read the sample element by element, take the full
 * pass without line skipping and never use row-split. Returns TOPK_ERR_BAD_ARG unless
 * 1 <= stride <= 65536 and 500 <= rho0 <= rho1 <= 4000. Process-wide; a captured graph
 * keeps the setting made before its capture. */
int topk_exact_set_proposal(int32_t stride, int32_t rho0_permille, int32_t rho1_permille);

/* Admission depth of rows whose sample is read one element per period (no passage
 * defines it; it is this library's addition to the pages' tau0 / tau1 fallback, [Cx]
 * section "采样不是处处都该开"). Such a row's single full pass admits every key at or
 * above tau_a, the sample key of rank ceil(T_A n_s / L) with T_A = rho_a * K (thousandths
 * of K), instead of stopping at tau1; C(tau0) and C(tau1) are counted among the admitted
 * keys afterwards, so the statistics still name the threshold that certifies each row, and
 * a row with C(tau1) < K <= C(tau_a) is finished without reading it again. T_A applies only
 * where T1 < T_A < T2 and T_A <= 9/16 of the 8192-slot candidate buffer, and in calls of at
 * most one row per resident workgroup (where a row's recovery would lengthen the call);
 * elsewhere (and for line-sampled rows, whose sample is 32 keys per period) admission stays
 * at tau1.
 * rho_a = 0 turns the deeper admission off (every row admits at tau1, as on the pages);
 * -1 restores the default 2250. Every setting gives an exact result. Returns
 * TOPK_ERR_BAD_ARG unless rho_a is -1, 0 or in [1000, 8000]. Process-wide; a captured
 * graph keeps the setting made before its capture. */
int topk_exact_set_admission(int32_t rhoa_permille);

/* Measurement hook (no passage defines it; it serves the per-kernel timing of the
 * roofline report beside the pages' per-call timing, [Cx] section "什么叫精确，时间怎么量"):
 * arms a one-shot timing of the next topk_exact call made on this host thread. That call records `start` on its stream just before its first
 * selector kernel and `stop` just after its last one, before the exact-recovery
 * kernels, so hipEventElapsedTime(start, stop) is the selector kernels' device time.
 * The events belong to the caller, were created on the current device with timing
 * enabled, and must stay alive until they have completed. A call under stream capture
 * records nothing and leaves the hook armed; (NULL, NULL) disarms it. Returns
 * TOPK_ERR_NULL_POINTER if exactly one event is NULL. */
int topk_exact_time_next_call(hipEvent_t start, hipEvent_t stop);

/* Measurement hook: per-row phase times (no passage defines the hook; it measures what
 * the pages report about the mechanism, [Cx] section "采样不是处处都该开": the time of the
 * sampled proposal against an exact one, the cost of the nested fallback and of exact
 * recovery per affected row). While armed, every topk_exact call of at most `rows` rows
 * outside stream capture writes, for each row r, 8 words at buf[8 r ...]: device
 * wall-clock stamps when its workgroup starts it [0], has read its sample [1], has
 * selected tau0 / tau1 / tau2 [2], has finished the full-row pass [3], has committed it
 * or handed it to the recovery kernels [4], and when its exact recovery finished [5];
 * [6] = path code (1 sentinel, 2 direct, 3 tau0, 4 tau1, 5 recovered in place, 6 queued
 * for the recovery kernels, 7 forced recovery; +128 for row-split rows, whose stamps [0]
 * and [4] bracket the final per-row kernel) | XCC id << 8 | hardware wave id << 32;
 * [7] = C(tau1) | C(tau0) << 32. Stamps a row's path does not reach are left as they
 * were (clear the buffer first). buf is device memory of [rows][8] uint64 owned by the
 * caller, kept alive while armed; (NULL, 0) disarms. wall_clock_khz (host, may be NULL)
 * receives the stamp frequency of the current device. Process-wide. Returns TOPK_OK,
 * TOPK_ERR_BAD_ARG (buf and rows not both set or both empty) or TOPK_ERR_HIP. */
int topk_exact_record_phases(uint64_t* buf, int64_t rows, int64_t* wall_clock_khz);

/* Text of the last error raised on this host thread ("" if none). A library utility; no
 * passage defines it. */
const char* topk_exact_last_error(void);

/* Bandwidth probe (a measurement aid that no passage defines; the measured read ceiling
 * reported beside the 8 TB/s peak, not part of the selection): reads n floats from
 * `x` (device, 16-byte aligned) with the same 128-bit non-temporal loads as the selector's
 * full-row pass, one workgroup per consecutive 4 MiB chunk, and writes one float per
 * workgroup into `sink` (device, >= 4096 floats; workgroup b writes slot b mod 4096) so the
 * reads cannot be elided. Used to report a measured HBM read ceiling next to the peak. */
int topk_stream_read_probe(const float* x, int64_t n, float* sink, hipStream_t stream);

/* FP8 indexer score producer: the score matrix the selector consumes, made on the GPU so
 * that scoring and selection can be chained on one stream and captured into one graph
 * (page "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K", section "框架轨迹": the
 * selector runs behind an FP8 multi-query attention score kernel in one graph). For every
 * query row t and key s it writes the DSA indexer score of page "LiteTopK: Exploiting the
 * Curse of Dimensionality for a Fused Indexer-TopK Kernel ..." (section 核心公式, Eq. (1)):
 *     out[t][s] = sum_{h < H} w[t][h] * max(0, sum_{d < D} q[t][h][d] * k[s][d])   for s < L_t
 *     out[t][s] = -inf                                                            for s >= L_t
 * with L_t = clamp(row_len[t], 0, S).
 *   q        device, [T][H][D] bytes, OCP FP8 E4M3 codes (row-major), 16-byte aligned.
 *   k        device, [S][D] bytes, OCP FP8 E4M3 codes (row-major), 16-byte aligned.
 *   w        device, [T][H] float32 head weights, 16-byte aligned.
 *   row_len  device, [T] int32 valid lengths (the selector's row_len).
 *   T, S     T >= 0 query rows, 1 <= S <= INT32_MAX - 4096 keys (the selector's N_alloc).
 *   H, D     H in {16, 32, 48, 64} heads, D = 128 (head dimension).
 *   out      device, row-major [T][S] float32; every element is written.
 *   stream   the kernel is enqueued here; no allocation or synchronization (capturable).
 * Products of E4M3 values are exact. The matrix cores add them in groups of 8 adjacent
 * d, truncating each product toward zero to a multiple of 2^(X - 13), X the largest
 * exponent sum e_q + e_k of the group's nonzero products (e: unbiased E4M3 exponent, -6
 * for subnormals); the group sums and the weighted sum over heads round in float32. Each
 * element is therefore within sum_h |w[t][h]| * sum_d (|p_d| mod 2^(X_g(d) - 13)) +
 * (D / 8 + H + 4) * 2^-24 * sum_h |w[t][h]| * sum_d |p_d| of the exact value, p_d =
 * q[t][h][d] * k[s][d] (no truncation loss when every product's exponent sum is within 7 of
 * its group's largest, as for typical data). NaN codes (S.1111.111)
 * are outside the contract (the result is unspecified). Returns TOPK_OK (T == 0 is a no-op), TOPK_ERR_BAD_SHAPE,
 * TOPK_ERR_BAD_ARG (H, D or alignment), TOPK_ERR_NULL_POINTER or TOPK_ERR_HIP, before
 * anything is enqueued except for TOPK_ERR_HIP. */
int topk_indexer_scores(const uint8_t* q, const uint8_t* k, const float* w, const int32_t* row_len,
                        int64_t T, int64_t S, int32_t H, int32_t D, float* out, hipStream_t stream);

/* The score + select chain in one call: topk_indexer_scores into `scores` (device,
 * [T][S] float32, caller-owned), then topk_exact(scores, row_len, T, S, K, out_idx,
 * sentinel) on the same stream, so one capture holds both (page "几何平均快 1.55 倍，但短行采样会输：
 * 腾讯怎么测精确 Top-K", section "框架轨迹": the selector behind an FP8 score kernel in one
 * graph). Arguments as in the two calls. Every host-side check of both (shapes, H, D, K,
 * sentinel, pointers, alignment, the workspace under capture) runs before anything is
 * enqueued; T == 0 is a no-op. */
int topk_indexer_topk(const uint8_t* q, const uint8_t* k, const float* w, const int32_t* row_len,
                      int64_t T, int64_t S, int32_t H, int32_t D, int32_t K, float* scores,
                      int32_t* out_idx, int32_t sentinel, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TOPK_EXACT_H */
