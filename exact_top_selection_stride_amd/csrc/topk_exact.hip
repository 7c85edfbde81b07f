// topk_exact.hip -- gfx950 (CDNA4, wave64) kernels and host dispatch for the
// sample-guided exact Top-K selector declared in include/topk_exact.h.
//
// Pages cited (by title):
//   [Cx] "几何平均快 1.55 倍，但短行采样会输：腾讯怎么测精确 Top-K"
//   [PD] "腾讯|长上下文稀疏注意力前K精确选择:20种配置平均加速1.55倍"
//   [AX] "Sample-Guided Exact Top-K Selection for Long-Context Sparse Attention"
//        (arxivdaily abstract page)
//
// Per row of the score matrix (one 512-thread workgroup works on a row at a time):
//   1. Rows with L <= K write 0..L-1 and the sentinel; no score is read
//      ([Cx] section "什么叫精确，时间怎么量").
//   2. Short rows (direct-exact, [Cx] section "采样不是处处都该开": exact
//      proposals win on short rows) are staged in LDS as order keys and
//      selected exactly there: one HBM read.
//   3. Longer rows take the sampled path ([PD] question 2, Fig. 4):
//      a. the fixed-stride view x[j*128] proposes tau0 (target 1.5K
//         candidates) and the nested, wider tau1 (target 1.75K) as ranks of
//         the sample ([Cx] section "采样不是处处都该开"; [PD] question 2). On
//         the long rows the sampled 128-byte lines are read whole, and the
//         full pass skips those whose maximum is below tau1 (line sampling,
//         below);
//      b. one mandatory full-row pass reads the row with 128-bit non-temporal
//         loads, admits keys >= tau1 into an LDS candidate buffer (per-lane
//         counts, one slot reservation per wave and batch), counts C(tau0)
//         and C(tau1), and builds the first radix histogram of the admitted
//         keys ([PD] question 2, Fig. 4 stage 2; [AX]);
//      c. certification: C(tau0) >= K, else C(tau1) >= K (the nested set is
//         already in LDS, so this fallback rereads nothing), else exact
//         full-row recovery; a candidate overflow also goes to recovery.
//         Nothing is written before this decision ([PD] question 2; [AX]);
//      d. refinement on the unresolved boundary only: bins above the bin that
//         holds rank K are committed at once, that bin's candidates move to a
//         small frontier buffer, where the K-th key is found exactly (rank
//         counting, or radix digits narrowing the bin) ([PD] question 2, Fig. 4
//         stage 3).
//   4. Exact full-row recovery is a radix select over the whole row, run after
//      the selector by three small kernels that spread the queued rows over the
//      GPU: a histogram pass, a pass that commits every key above the boundary
//      bin and collects that bin, and a finish step per row.
// Rows map to workgroups by shape ([AX]; [PD] question 2): several workgroups
// per row for few long rows (row-split), a persistent grid pulling rows from a
// device ticket for many long rows, one workgroup per row otherwise.
//
// Keys: a float's 32-bit pattern u maps to key(u) = u ^ (sign ? 0xFFFFFFFF :
// 0x80000000), whose unsigned order is IEEE totalOrder. The hot loop never
// builds keys: admission key(u) >= key(tau1) is a single signed compare of u
// (tau1 >= +0) or unsigned compare (tau1 <= -0). No floating-point arithmetic
// happens anywhere on the path.
//
// Code conventions: the workgroup's LDS state is one file-scope __shared__
// object, and score/output rows are handled through address-space-1 (global)
// pointers, so every helper, inlined anywhere, compiles its accesses to ds_* /
// global_* instructions (never flat ones). The whole per-row path is inlined
// into each kernel: an out-of-line call per row would save and restore its
// callee-saved registers through scratch memory for every row.

#include "topk_exact.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#define GLB __attribute__((address_space(1)))

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const GLB uint32_t* grow_t;   // a row of score bit patterns
typedef GLB int32_t* gout_t;          // a row of output indices

// A row's output: its K index slots and, for the sorted output, the selected keys in the
// same slots (so that the sort needs no second read of the scores). Every selected
// element is written through put().
struct RowOut {
  gout_t idx;
  GLB uint32_t* key;  // null unless the keys are wanted
  __device__ __forceinline__ void put(uint32_t slot, uint32_t index, uint32_t k) const {
    idx[slot] = (int32_t)index;
    if (key != nullptr) key[slot] = k;
  }
};

constexpr int BLOCK = 512;            // threads per workgroup (8 waves of 64)
constexpr int WAVE = 64;
constexpr int NWAVES = BLOCK / WAVE;
constexpr int NB_BITS = 11;
constexpr int NB = 1 << NB_BITS;      // radix histogram bins
constexpr int CAP = 8192;             // candidate (index, key) pairs in LDS
constexpr int KEYS_CAP = 2 * CAP;     // keys-only capacity of the same region
constexpr int FL_CAP = 512;           // frontier (index, key) pairs
constexpr uint32_t FL_RANK_MAX = 64;  // frontiers up to this size are resolved by rank counting
constexpr uint32_t STRIDE = 128;      // sample stride s
constexpr int UNROLL = 4;             // 128-bit loads per thread per batch (whole-row walks)
constexpr int PASS_UNROLL = 6;        // 128-bit loads per lane per batch of the fused pass
constexpr uint32_t DIRECT_MAX_DEFAULT = 16384;
constexpr uint32_t QMAX = 256;        // rows queued for cooperative recovery per call (workspace)
constexpr uint32_t REC_SEG = 16384;   // elements per recovery work item (rows wider than 256K)
constexpr uint32_t REC_SEG_SHORT = 4096;  // ... and for rows of up to 256K
constexpr int64_t REC_SHORT_MAX_N = 262144;
constexpr uint32_t INPLACE_MAX = 65536;        // rows up to this length are recovered in place,
constexpr uint32_t INPLACE_MAX_SPLIT = 262144; // ... and up to this one in row-split calls
constexpr int64_t ROWSPLIT_MIN_N = 65536;  // auto row-split only for rows at least this wide
constexpr uint32_t KEY_MAX = 0xFFFFFFFFu;

static_assert(NB % BLOCK == 0, "bins per thread must be integral");
// K = 2048 is the operating point of the method; larger K (up to TOPK_K_MAX) keeps
// the same targets, so tau1 admits about 1.75 K of the CAP slots and the rows whose
// candidates overflow them take exact recovery.
static_assert(TOPK_K_MAX * 7 / 4 + 1 <= CAP, "candidate buffer must hold the tau1 target");
static_assert(FL_CAP <= BLOCK, "frontier lists are ranked one element per thread");
static_assert(TOPK_K_MAX <= 8 * BLOCK, "the sorted output holds at most 8 entries per thread");

struct Control {
  uint32_t row_ticket;   // next row of the persistent row loop
  uint32_t done_ticket;  // workgroups that left the row loop
  uint32_t qcount;       // rows queued for cooperative recovery in this call
  uint32_t rec_done;     // workgroups that finished the recovery collect kernel
  uint32_t pad[28];
  unsigned long long stats[TOPK_STAT_COUNT];
};

// One row queued for cooperative exact recovery. Written by the workgroup that
// queues the row; the histogram, counters and candidates are filled by the
// recovery kernels.
// Recovery slot modes. REC_WINDOW: the K-th key is known to lie in [bin_lo, bin_hi]
// (the row's own pass located it), so the collect and finish kernels complete the row
// alone. REC_HIST: nothing is known; the histogram kernel first bins the whole row.
constexpr uint32_t REC_HIST = 0u, REC_WINDOW = 1u;

struct RecSlot {
  uint32_t row;
  uint32_t L;
  uint32_t lo, hi;       // key range binned by the histogram (REC_HIST); fallback range (REC_WINDOW)
  uint32_t out_gt;       // next output slot for keys above the boundary bin
  uint32_t cnt;          // candidates collected from the boundary bin (all, even past CAP)
  uint32_t bin_above;    // keys above the boundary bin
  uint32_t bin_count;    // keys in the boundary bin (REC_HIST)
  uint32_t bin_lo, bin_hi;
  uint32_t mode;         // REC_HIST or REC_WINDOW
  uint32_t commit;       // REC_WINDOW: the collect kernel commits the keys above bin_hi
  uint32_t pad[20];
  uint32_t hist[NB];
  uint32_t cand_idx[CAP];
  uint32_t cand_key[CAP];
};

struct Params {
  const float* scores;
  const int32_t* row_len;
  int32_t* out;
  Control* ctl;
  uint32_t M;
  uint32_t N;
  uint32_t K;
  int32_t sentinel;
  uint32_t T0;          // primary candidate target, ceil(1.5 K) by default
  uint32_t T1;          // secondary candidate target, ceil(1.75 K) by default
  uint32_t T2;          // threshold for in-place recovery of underfilled rows (a deeper target)
  uint32_t TA;          // admission target of element-sampled rows (T1 <= TA <= T2)
  uint32_t inplace_max; // rows up to this length needing exact recovery are recovered in place
  uint32_t stride;      // sample stride s, 128 by default
  uint32_t line_min;    // sampled rows with at least this many sample lines use line sampling
  uint32_t direct_max;  // auto mode: rows up to this length take the direct path
  int32_t mode;
  RecSlot* rec;         // qmax recovery slots
  uint32_t qmax;        // rows a call can queue for cooperative recovery
  struct RowSplitState* rs;  // per-row state of the row-split kernels
  uint32_t ps;          // row-split: workgroups per row sampling
  uint32_t pp;          // row-split: workgroups per row passing
  uint32_t pass_taus;   // row-split: each passing workgroup selects the row's taus itself
  uint32_t split_elem;  // row-split: ... from the row's element sample, read by itself (no sample kernel)
  unsigned long long* phase;  // per-row phase record (PHASE_WORDS per row), or null
  uint32_t* okey;       // [M][K] selected keys beside out (sorted output), or null
  uint32_t sort_rows;   // sorted output: each row is sorted by its workgroup once complete
  float* oval;          // sorted output values (with sort_rows), or null
};

__device__ __forceinline__ RowOut row_out(const Params& p, uint32_t row) {
  RowOut o;
  o.idx = (gout_t)(p.out) + (size_t)row * p.K;
  o.key = p.okey != nullptr ? (GLB uint32_t*)(p.okey) + (size_t)row * p.K : nullptr;
  return o;
}

struct alignas(16) Smem {
  uint32_t buf[2 * CAP];       // candidates: idx in [0,CAP), key in [CAP,2CAP); or keys only
  uint32_t hist[NB];
  uint32_t fl_idx[FL_CAP];
  uint32_t fl_key[FL_CAP];
  uint32_t wtmp[NWAVES];
  uint32_t cnt;                // admitted / collected count
  uint32_t cnt0;               // admitted keys >= tau0 (counted from the list after the pass)
  uint32_t cnt1;               // admitted keys >= tau1 (likewise)
  uint32_t fl_cnt;
  uint32_t out_gt;             // output slots taken by keys above the threshold
  uint32_t out_tie;            // output slots taken by keys equal to the threshold
  uint32_t pass_next;          // next batch of the full-row pass to claim
  uint32_t mn, mx;
  uint32_t sel_bin, sel_above;
  uint32_t bcast;              // block-wide broadcast of a value read by thread 0
  uint32_t bcast2;
  uint32_t queued;             // the row was handed to the recovery kernels (sorted output)
  int32_t row;
};

__shared__ Smem g_s;  // the selector workgroup's LDS state

// ---------------------------------------------------------------- primitives

__device__ __forceinline__ uint32_t key_of_bits(uint32_t u) {
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

__device__ __forceinline__ uint32_t mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ u32x4 load4(grow_t p) { return *reinterpret_cast<const GLB u32x4*>(p); }

// Streaming load for the full-row pass: the non-temporal hint keeps the single-use
// row data from displacing cached lines (measured on MI355X: ~7.0 TB/s for a plain
// read with the hint against ~6.2 TB/s without). Loads whose lines are read again
// (the sampled lines, re-read when hot) stay ordinary.
__device__ __forceinline__ u32x4 load4_stream(grow_t p) {
  return __builtin_nontemporal_load(reinterpret_cast<const GLB u32x4*>(p));
}

__device__ __forceinline__ u32x4 splat4(uint32_t v) { return u32x4{v, v, v, v}; }

// Reserves consecutive slots of an LDS counter for the lanes whose pred is set, one
// atomic per wave. Every active lane of the wave must reach it.
__device__ __forceinline__ uint32_t wave_reserve(bool pred, uint32_t* counter) {
  const uint64_t m = __ballot(pred);
  uint32_t base = 0;
  if (m != 0) {
    const int leader = __builtin_ctzll(m);
    uint32_t b = 0;
    if ((int)lane_id() == leader) b = atomicAdd(counter, (uint32_t)__popcll(m));
    base = (uint32_t)__builtin_amdgcn_readlane((int)b, leader);
  }
  return base + mbcnt64(m);
}

// Reserves cnt consecutive slots of an LDS counter for every lane (cnt < 2^NBITS) with
// one atomic per wave: the wave's prefix counts come from the ballots of the count's
// bits. Returns this lane's first slot. Every active lane of the wave must reach it.
template <int NBITS>
__device__ __forceinline__ uint32_t wave_reserve_n(uint32_t cnt, uint32_t* counter) {
  uint32_t total = 0, before = 0;
#pragma unroll
  for (int bit = 0; bit < NBITS; ++bit) {
    const uint64_t m = __ballot((cnt >> bit) & 1u);
    total += (uint32_t)__popcll(m) << bit;
    before += mbcnt64(m) << bit;
  }
  uint32_t b = 0;
  if (total != 0) {
    const int leader = __builtin_ctzll(__ballot(true));
    if ((int)lane_id() == leader) b = atomicAdd(counter, total);
    b = (uint32_t)__builtin_amdgcn_readfirstlane(b);
  }
  return b + before;
}

// Per-thread item counts of LDS lists walked as i = t, t + BLOCK, ... or four entries at
// a time (i = 4 t, 4 t + 4 BLOCK, ...): at most 32 for lists of up to 16384 entries.
constexpr int LIST_BITS = 6;
static_assert((KEYS_CAP + BLOCK - 1) / BLOCK < (1 << LIST_BITS), "per-thread list counts fit LIST_BITS");
static_assert(CAP < 0x10000, "two per-wave counts of admitted keys share one word");

// Cross-lane steps through DPP (GFX9 family controls): row_shr:n moves each lane's value
// n lanes up within its row of 16; row_bcast:15 / row_bcast:31 pass lane 15 / 31 on to
// the following row(s), which the row mask selects. Lanes that receive nothing keep
// `old`. Each step is one VALU instruction, where a shuffle is an LDS round trip.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
}
constexpr int DPP_QUAD_SWAP1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_SWAP2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROW_SHL = 0x100;      // + n, n in 1..15
constexpr int DPP_ROW_SHR = 0x110;      // + n, n in 1..15
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

// Inclusive scan over the 64 lanes of a wave (every lane active): a within-row
// Kogge-Stone scan, then row totals carried into rows 1, 3 and 2, 3.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<DPP_ROW_SHR + 1>(0u, v);
  v += dpp<DPP_ROW_SHR + 2>(0u, v);
  v += dpp<DPP_ROW_SHR + 4>(0u, v);
  v += dpp<DPP_ROW_SHR + 8>(0u, v);
  v += dpp<DPP_ROW_BCAST15, 0xa>(0u, v);
  v += dpp<DPP_ROW_BCAST31, 0xc>(0u, v);
  return v;
}

// Minimum / maximum over the wave (every lane active), returned to every lane: the
// same scan structure leaves the result in lane 63.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp<DPP_ROW_SHR + 1>(KEY_MAX, v));
  v = min(v, dpp<DPP_ROW_SHR + 2>(KEY_MAX, v));
  v = min(v, dpp<DPP_ROW_SHR + 4>(KEY_MAX, v));
  v = min(v, dpp<DPP_ROW_SHR + 8>(KEY_MAX, v));
  v = min(v, dpp<DPP_ROW_BCAST15, 0xa>(KEY_MAX, v));
  v = min(v, dpp<DPP_ROW_BCAST31, 0xc>(KEY_MAX, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, WAVE - 1);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp<DPP_ROW_SHR + 1>(0u, v));
  v = max(v, dpp<DPP_ROW_SHR + 2>(0u, v));
  v = max(v, dpp<DPP_ROW_SHR + 4>(0u, v));
  v = max(v, dpp<DPP_ROW_SHR + 8>(0u, v));
  v = max(v, dpp<DPP_ROW_BCAST15, 0xa>(0u, v));
  v = max(v, dpp<DPP_ROW_BCAST31, 0xc>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, WAVE - 1);
}

// Exchange with lane ^ J across the wave: DPP within rows of 16 lanes for J <= 8 (quad
// permutes for 1 and 2; a shift each way, limited to the banks it serves, for 4 and 8),
// a permute through the LDS crossbar for 16 and 32.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) return dpp<DPP_QUAD_SWAP1>(0u, v);
  else if constexpr (J == 2) return dpp<DPP_QUAD_SWAP2>(0u, v);
  else if constexpr (J == 4) return dpp<DPP_ROW_SHR + 4, 0xf, 0xa>(dpp<DPP_ROW_SHL + 4, 0xf, 0x5>(0u, v), v);
  else if constexpr (J == 8) return dpp<DPP_ROW_SHR + 8, 0xf, 0xc>(dpp<DPP_ROW_SHL + 8, 0xf, 0x3>(0u, v), v);
  else return (uint32_t)__shfl_xor((int)v, J);
}

// One bitonic stage over the wave: lane pairs (l, l ^ J) compare-exchange, the lower lane
// keeping the larger value where bit KB of the lane is clear (descending runs).
template <int KB, int J>
__device__ __forceinline__ uint32_t bitonic_step(uint32_t v) {
  const uint32_t p = lane_xor<J>(v);
  const uint32_t l = lane_id();
  const bool keep_max = ((l & (uint32_t)J) == 0u) == ((l & (1u << KB)) == 0u);
  return keep_max ? max(v, p) : min(v, p);
}

// The wave's 64 values sorted in descending order across its lanes (lane 0 the largest).
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t v) {
  v = bitonic_step<1, 1>(v);
  v = bitonic_step<2, 2>(v);  v = bitonic_step<2, 1>(v);
  v = bitonic_step<3, 4>(v);  v = bitonic_step<3, 2>(v);  v = bitonic_step<3, 1>(v);
  v = bitonic_step<4, 8>(v);  v = bitonic_step<4, 4>(v);  v = bitonic_step<4, 2>(v);  v = bitonic_step<4, 1>(v);
  v = bitonic_step<5, 16>(v); v = bitonic_step<5, 8>(v);  v = bitonic_step<5, 4>(v);  v = bitonic_step<5, 2>(v);
  v = bitonic_step<5, 1>(v);
  v = bitonic_step<6, 32>(v); v = bitonic_step<6, 16>(v); v = bitonic_step<6, 8>(v);  v = bitonic_step<6, 4>(v);
  v = bitonic_step<6, 2>(v);  v = bitonic_step<6, 1>(v);
  return v;
}

// Smallest shift such that span >> shift fits in NB bins (at most 21).
__device__ __forceinline__ uint32_t shift_for(uint32_t span) {
  if (span < (uint32_t)NB) return 0;
  return (32u - (uint32_t)__clz(span)) - NB_BITS;
}

__device__ __forceinline__ void stat_add(Control* ctl, int slot) {
  atomicAdd(&ctl->stats[slot], 1ull);
}

// Per-row phase record (measurement hook, armed by topk_exact_record_phases): device
// wall-clock stamps of the row's phases, its path and where it ran. Written by thread 0
// of the workgroup that owns the phase; nothing is written while the hook is disarmed.
constexpr int PHASE_WORDS = 8;
enum : int {
  PH_START = 0,      // the row's workgroup starts on it
  PH_SAMPLED = 1,    // sample read, min/max known
  PH_PROPOSED = 2,   // tau0 / tau1 / tau_a / tau2 selected
  PH_PASSED = 3,     // fused full-row pass done
  PH_END = 4,        // committed, or handed to the recovery kernels
  PH_RECOVERED = 5,  // exact recovery done (in place, or by the recovery finish kernel)
  PH_WHERE = 6,      // path code | XCC id << 8 | hardware wave id << 32
  PH_COUNTS = 7,     // C(tau1) | C(tau0) << 32 (certified rows), else the admitted count
};
enum : uint32_t {
  PATH_SENTINEL = 1, PATH_DIRECT = 2, PATH_TAU0 = 3, PATH_TAU1 = 4, PATH_RECOVER_INPLACE = 5,
  PATH_RECOVER_QUEUED = 6, PATH_FORCED_RECOVERY = 7, PATH_TAUA = 8, PATH_SPLIT_FLAG = 0x80,
};

__device__ __forceinline__ void phase_put(unsigned long long* ph, uint32_t row, int slot, unsigned long long v) {
  if (ph != nullptr && threadIdx.x == 0) ph[(size_t)row * PHASE_WORDS + slot] = v;
}

__device__ __forceinline__ void phase_mark(unsigned long long* ph, uint32_t row, int slot) {
  if (ph != nullptr && threadIdx.x == 0) ph[(size_t)row * PHASE_WORDS + slot] = (unsigned long long)wall_clock64();
}

// Records the row's path with the XCC and hardware wave id (HW_ID register) it ran on.
__device__ __forceinline__ void phase_path(unsigned long long* ph, uint32_t row, uint32_t code) {
  if (ph != nullptr && threadIdx.x == 0) {
    const uint32_t hw = (uint32_t)__builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID, 32 bits
    const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | 20);  // XCC_ID, 4 bits
    ph[(size_t)row * PHASE_WORDS + PH_WHERE] =
        (unsigned long long)(code | (xcc << 8)) | ((unsigned long long)hw << 32);
  }
}

// Folds per-thread min/max into s.mn / s.mx (initialised by the caller before a
// barrier). Ends with a barrier.
__device__ __forceinline__ void block_minmax(uint32_t mn, uint32_t mx) {
  Smem& s = g_s;
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane_id() == 0) {
    atomicMin(&s.mn, mn);
    atomicMax(&s.mx, mx);
  }
  __syncthreads();
}

// Finds the bin b holding rank r (1-based, counted from the top) of s.hist and the
// count of entries in bins above it. Requires 1 <= r <= sum(hist). Result in
// s.sel_bin / s.sel_above; starts and ends with a barrier-protected section.
__device__ void block_find_bin(uint32_t r) {
  Smem& s = g_s;
  constexpr int PER = NB / BLOCK;
  const uint32_t t = threadIdx.x;
  uint32_t h[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    h[j] = s.hist[t * PER + j];
    sum += h[j];
  }
  uint32_t incl = wave_incl_scan(sum);
  const uint32_t w = t / WAVE;
  if (lane_id() == WAVE - 1) s.wtmp[w] = incl;
  if (t == 0) {
    s.sel_bin = 0;
    s.sel_above = 0;
  }
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    const uint32_t v = s.wtmp[i];
    before += ((uint32_t)i < w) ? v : 0u;
    total += v;
  }
  incl += before;
  const uint32_t above = total - incl;  // entries in bins owned by higher threads
  if (above < r && r <= above + sum) {
    uint32_t cum = above;
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      if (cum + h[j] >= r) {
        s.sel_bin = t * PER + j;
        s.sel_above = cum;
        break;
      }
      cum += h[j];
    }
  }
  __syncthreads();
}

// Exact rank selection by radix narrowing. `for_keys(f)` calls f(key) for every key
// of the set, block-cooperatively. Among the keys in [lo, hi], finds T = the r-th
// largest (1 <= r <= count in range) and gt = the number of them above T. Each
// round bins the range into NB buckets, keeps only the bucket holding rank r, and
// shrinks the range by 2^11, so at most three rounds run.
template <class ForKeys>
__device__ void select_rank(ForKeys&& for_keys, uint32_t r, uint32_t lo, uint32_t hi, uint32_t& T,
                            uint32_t& gt) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  gt = 0;
  for (;;) {
    const uint32_t sh = shift_for(hi - lo);
    for (uint32_t i = t; i < (uint32_t)NB; i += BLOCK) s.hist[i] = 0;
    __syncthreads();
    const uint32_t lo_ = lo, hi_ = hi;
    for_keys([&](uint32_t k) {
      if (k >= lo_ && k <= hi_) atomicAdd(&s.hist[(k - lo_) >> sh], 1u);
    });
    __syncthreads();
    block_find_bin(r);
    const uint32_t b = s.sel_bin, above = s.sel_above;
    r -= above;
    gt += above;
    const uint32_t blo = lo + (b << sh);
    if (sh == 0) {
      T = blo;
      break;
    }
    const uint32_t wdt = (1u << sh) - 1u;
    const uint32_t d = hi - blo;
    lo = blo;
    hi = blo + (d < wdt ? d : wdt);
  }
  __syncthreads();
}

// For a short key list in LDS (m <= BLOCK): thread i < m returns the number of keys
// ahead of keys[i] in the strict order (key descending, position ascending).
// keys must be 16-byte aligned: they are read four at a time, several reads in flight.
__device__ __forceinline__ uint32_t rank_in_list(const uint32_t* keys, uint32_t m) {
  const uint32_t i = threadIdx.x;
  if (i >= m) return KEY_MAX;
  const uint32_t ki = keys[i];
  auto ahead = [&](uint32_t kj, uint32_t j) -> uint32_t { return (kj > ki || (kj == ki && j < i)) ? 1u : 0u; };
  uint32_t r = 0, j = 0;
  const uint32_t m4 = m & ~3u;
#pragma unroll 4
  for (; j < m4; j += 4) {
    const u32x4 k4 = *reinterpret_cast<const u32x4*>(keys + j);
    r += ahead(k4.x, j) + ahead(k4.y, j + 1) + ahead(k4.z, j + 2) + ahead(k4.w, j + 3);
  }
  for (; j < m; ++j) r += ahead(keys[j], j);
  return r;
}

template <class F>
__device__ __forceinline__ void quad(const u32x4& v, uint32_t e, F&& f) {
  f(v.x, e);
  f(v.y, e + 1);
  f(v.z, e + 2);
  f(v.w, e + 3);
}

// Calls f(bits, index) for every element of x[0, L), block-cooperatively, with
// 128-bit loads for the aligned body. Lanes of a wave call f in lockstep (with
// trailing lanes masked off), so f may use wave-wide ballots.
template <class F>
__device__ void for_each_element(grow_t x, uint32_t L, F&& f) {
  const uint32_t t = threadIdx.x;
  uint32_t head = (uint32_t)((4u - ((uint32_t)((uintptr_t)x >> 2) & 3u)) & 3u);
  if (head > L) head = L;
  if (t < head) f(x[t], t);
  const uint32_t nv = (L - head) >> 2;
  grow_t body = x + head;
  const uint32_t per = BLOCK * UNROLL;
  uint32_t q0 = 0;
  for (; q0 + per <= nv; q0 += per) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) v[u] = load4(body + 4u * (q0 + u * BLOCK + t));
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) quad(v[u], head + 4u * (q0 + u * BLOCK + t), f);
  }
  for (uint32_t q = q0 + t; q < nv; q += BLOCK) quad(load4(body + 4u * q), head + 4u * q, f);
  const uint32_t tail0 = head + 4u * nv;
  if (t < L - tail0) f(x[tail0 + t], tail0 + t);
}

// Zeroes the per-row counters and the histogram; ends with a barrier.
__device__ __forceinline__ void reset_row_state() {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  for (uint32_t i = t; i < (uint32_t)NB; i += BLOCK) s.hist[i] = 0;
  if (t == 0) {
    s.cnt = 0;
    s.cnt0 = 0;
    s.cnt1 = 0;
    s.fl_cnt = 0;
    s.out_gt = 0;
    s.out_tie = 0;
    s.pass_next = 0;
    s.mn = KEY_MAX;
    s.mx = 0;
  }
  __syncthreads();
}

// Commits keys > T (slots continue from s.out_gt) and up to K - gt_total keys == T
// (slots gt_total + 0..) from a key list in LDS with indices idx (or the position).
__device__ __forceinline__ void commit_list(const uint32_t* keys, const uint32_t* idx, uint32_t n,
                                            uint32_t T, uint32_t gt_total, uint32_t K, RowOut out) {
  Smem& s = g_s;
  const uint32_t ties = K - gt_total;
  // Count this thread's keys of each kind, reserve their slots once per wave, then write.
  uint32_t ng = 0, ne = 0;
  for (uint32_t i = threadIdx.x; i < n; i += BLOCK) {
    const uint32_t k = keys[i];
    ng += k > T ? 1u : 0u;
    ne += k == T ? 1u : 0u;
  }
  uint32_t p = wave_reserve_n<LIST_BITS>(ng, &s.out_gt);
  uint32_t q = wave_reserve_n<LIST_BITS>(ne, &s.out_tie);
  if (ng + ne == 0) return;
  for (uint32_t i = threadIdx.x; i < n; i += BLOCK) {
    const uint32_t k = keys[i];
    if (k > T) {
      if (p < K) out.put(p, idx ? idx[i] : i, k);
      ++p;
    } else if (k == T) {
      if (q < ties && gt_total + q < K) out.put(gt_total + q, idx ? idx[i] : i, k);
      ++q;
    }
  }
}

// ------------------------------------------------------ exact full-row select

// Exact selection of K of x[0, L) read from global memory (L > K). [lo, hi] is a key
// range expected to hold the K-th key; bins clamp outside it, so any range is
// correct and a good one makes the boundary bin small. Pass 1 builds the
// histogram; pass 2 commits every key above the boundary bin and collects that bin
// into LDS; the bin is then resolved exactly. If the bin exceeds the LDS buffer,
// it is narrowed by further passes over the row instead.
__device__ __attribute__((noinline)) void exact_full_row(grow_t x, uint32_t L, uint32_t K, uint32_t lo,
                                                         uint32_t hi, RowOut out, Control* ctl) {
  Smem& s = g_s;
  reset_row_state();
  const uint32_t sh = shift_for(hi - lo);
  for_each_element(x, L, [&](uint32_t u, uint32_t) {
    const uint32_t k = key_of_bits(u);
    const uint32_t d = k < lo ? 0u : (k - lo) >> sh;
    atomicAdd(&s.hist[d < (uint32_t)(NB - 1) ? d : (uint32_t)(NB - 1)], 1u);
  });
  __syncthreads();
  block_find_bin(K);
  const uint32_t b = s.sel_bin, above = s.sel_above;
  const uint32_t cb = s.hist[b];
  const uint32_t need = K - above;
  const uint32_t braw = lo + (b << sh);
  const uint32_t blo = (b == 0) ? 0u : braw;
  const uint32_t wdt = (1u << sh) - 1u;
  const uint32_t bhi = (b == (uint32_t)(NB - 1)) ? KEY_MAX
                                                 : braw + ((KEY_MAX - braw) < wdt ? (KEY_MAX - braw) : wdt);
  const bool fits = cb <= (uint32_t)CAP;
  __syncthreads();
  for_each_element(x, L, [&](uint32_t u, uint32_t e) {
    const uint32_t k = key_of_bits(u);
    const bool g = k > bhi;
    const uint32_t p = wave_reserve(g, &s.out_gt);
    if (g && p < K) out.put(p, e, k);
    if (fits) {
      const bool in = k >= blo && k <= bhi;
      const uint32_t f = wave_reserve(in, &s.cnt);
      if (in && f < (uint32_t)CAP) {
        s.buf[f] = e;
        s.buf[CAP + f] = k;
      }
    }
  });
  __syncthreads();
  uint32_t T, gt2;
  if (fits) {
    const uint32_t* keys = &s.buf[CAP];
    select_rank([&](auto&& f) {
      for (uint32_t i = threadIdx.x; i < cb; i += BLOCK) f(keys[i]);
    }, need, blo, bhi, T, gt2);
    commit_list(keys, s.buf, cb, T, above + gt2, K, out);
  } else {
    if (threadIdx.x == 0) stat_add(ctl, TOPK_STAT_FRONTIER_WIDE);
    select_rank([&](auto&& f) {
      for_each_element(x, L, [&](uint32_t u, uint32_t) { f(key_of_bits(u)); });
    }, need, blo, bhi, T, gt2);
    const uint32_t gt_total = above + gt2;
    const uint32_t ties = K - gt_total;
    for_each_element(x, L, [&](uint32_t u, uint32_t e) {
      const uint32_t k = key_of_bits(u);
      const bool g = k > T && k <= bhi;
      const uint32_t p = wave_reserve(g, &s.out_gt);
      if (g && p < K) out.put(p, e, k);
      const bool q_ = k == T;
      const uint32_t q = wave_reserve(q_, &s.out_tie);
      if (q_ && q < ties && gt_total + q < K) out.put(gt_total + q, e, k);
    });
  }
}

// ---------------------------------------------------------- direct (in LDS)

// Direct exact selection of a short row: the row is staged in LDS as keys (one HBM
// read), its first histogram over [min, max] is built there, and the LDS list is
// refined like a certified candidate list (refine_list, below).
template <bool KEYS_ONLY, bool COUNT = false>
__device__ __forceinline__ void refine_list(uint32_t n, uint32_t K, uint32_t base, uint32_t sh, RowOut out,
                                            Control* ctl, uint32_t k0 = 0u, uint32_t k1 = 0u);

__device__ __forceinline__ void direct_exact(grow_t x, uint32_t L, uint32_t K, RowOut out, Control* ctl) {
  Smem& s = g_s;
  uint32_t mn = KEY_MAX, mx = 0;
  for_each_element(x, L, [&](uint32_t u, uint32_t e) {
    const uint32_t k = key_of_bits(u);
    s.buf[e] = k;
    mn = min(mn, k);
    mx = max(mx, k);
  });
  block_minmax(mn, mx);
  const uint32_t lo = s.mn, hi = s.mx;
  const uint32_t sh = shift_for(hi - lo);
  for (uint32_t i = 4u * threadIdx.x; i < L; i += 4u * BLOCK) {
    // four keys per 16-byte LDS read; entries from L on are stale and skipped
    const u32x4 k4 = *reinterpret_cast<const u32x4*>(&s.buf[i]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + (uint32_t)u < L) atomicAdd(&s.hist[(k4[u] - lo) >> sh], 1u);
  }
  __syncthreads();
  refine_list<true>(L, K, lo, sh, out, ctl);
}

// ---------------------------------------------------------------- sampled path

struct PassCtx {
  uint32_t thr;    // raw-bit admission threshold (see admits)
  uint32_t akey;   // admission key (tau1, or the deeper admission rank): admitted keys are >= it
  uint32_t sh;     // first-histogram shift
};

// key(u) >= the admission key, evaluated on raw bits: for a threshold >= +0 it is a
// signed compare against its bits, for one <= -0 an unsigned <= against its bits.
template <bool POS>
__device__ __forceinline__ bool admits(uint32_t u, uint32_t thr) {
  return POS ? ((int32_t)u >= (int32_t)thr) : (u <= thr);
}

// A value that never passes admits<POS> (an admission key != 0 is required for NEG).
template <bool POS>
constexpr uint32_t never_admitted() { return POS ? 0x80000000u : 0xFFFFFFFFu; }

// Candidate formation for one element slot across the wave: ballot, one LDS atomic
// per wave for the base slot, prefix count for each lane's slot and histogram update.
// Every active lane of the wave must reach it.
template <bool POS>
__device__ __forceinline__ void admit_one(bool valid, uint32_t u, uint32_t e, const PassCtx c) {
  Smem& s = g_s;
  const bool pred = valid && admits<POS>(u, c.thr);
  const uint64_t m = __ballot(pred);
  if (m == 0) return;
  const int leader = __builtin_ctzll(m);
  uint32_t b = 0;
  if ((int)lane_id() == leader) b = atomicAdd(&s.cnt, (uint32_t)__popcll(m));
  const uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)b, leader) + mbcnt64(m);
  if (pred) {
    const uint32_t k = key_of_bits(u);
    if (pos < (uint32_t)CAP) {
      s.buf[pos] = e;
      s.buf[CAP + pos] = k;
    }
    const uint32_t d = (k - c.akey) >> c.sh;
    atomicAdd(&s.hist[d < (uint32_t)(NB - 1) ? d : (uint32_t)(NB - 1)], 1u);
  }
}

// Candidate formation for NQ quads per lane (element e[q] + i holds v[q][i]; values
// that must not be admitted are masked to never_admitted beforehand). Each lane counts
// its admitted elements; the wave's prefix counts come from the ballots of the count's
// bits, so one LDS atomic per wave reserves the slots of the whole batch and each lane
// then writes its candidates to consecutive slots. Every active lane of the wave must
// reach it.
template <bool POS, int NQ>
__device__ __forceinline__ void admit_batch(const u32x4 (&v)[NQ], const uint32_t (&e)[NQ], const PassCtx c) {
  Smem& s = g_s;
  constexpr int NBITS = 32 - __builtin_clz(4u * NQ);  // bits of a count in [0, 4 NQ]
  uint32_t n = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    n += admits<POS>(v[q].x, c.thr) ? 1u : 0u;
    n += admits<POS>(v[q].y, c.thr) ? 1u : 0u;
    n += admits<POS>(v[q].z, c.thr) ? 1u : 0u;
    n += admits<POS>(v[q].w, c.thr) ? 1u : 0u;
  }
  uint32_t pos = wave_reserve_n<NBITS>(n, &s.cnt);
  if (n == 0) return;
  // Slots are addressed in bytes, and those past the buffer are clamped onto its last
  // slot: a row that overflows is recovered from the histogram alone, so what that slot
  // then holds is never read. With POS every admitted value is >= +0, whose order key is
  // its bits with the top bit set, and key - akey = bits - (akey without its top bit).
  uint32_t pb = 4u * pos;
  const uint32_t ubase = c.akey & 0x7FFFFFFFu;
  auto one = [&](uint32_t u, uint32_t idx) {
    if (admits<POS>(u, c.thr)) {
      const uint32_t at = pb < 4u * (CAP - 1) ? pb : 4u * (CAP - 1);
      const uint32_t k = POS ? (u | 0x80000000u) : key_of_bits(u);
      *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(s.buf) + at) = idx;
      *reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(s.buf + CAP) + at) = k;
      const uint32_t d = (POS ? (u - ubase) : (k - c.akey)) >> c.sh;
      atomicAdd(&s.hist[d < (uint32_t)(NB - 1) ? d : (uint32_t)(NB - 1)], 1u);
      pb += 4u;
    }
  };
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    one(v[q].x, e[q]);
    one(v[q].y, e[q] + 1u);
    one(v[q].z, e[q] + 2u);
    one(v[q].w, e[q] + 3u);
  }
}

template <bool POS>
__device__ __forceinline__ void admit_quad(const u32x4& v, uint32_t e, const PassCtx c) {
  const u32x4 vv[1] = {v};
  const uint32_t ee[1] = {e};
  admit_batch<POS, 1>(vv, ee, c);
}

// The mandatory full-row pass: certification counts, candidate compaction and the
// first histogram, fused. The row body is cut into batches of PASS_UNROLL 128-bit loads
// per lane of one wave (6 KB); each wave claims its next batch from an LDS counter and
// issues that batch's loads before it examines the current one, so it keeps up to
// 2 x PASS_UNROLL loads in flight. Waves of a workgroup do not issue at the same rate (the
// older ones are served first); claiming batches dynamically keeps every wave busy
// until the row's last batch, where a fixed split of the row left the fast waves
// waiting at the closing barrier while the slow ones finished their share with fewer
// loads in flight. The counter s.pass_next is zeroed by reset_row_state.
//
// With SKIP, the row's sampled lines were read whole by the line sampler, and bit P
// of the LDS bitmap s.fl_idx says whether the sampled line of period P (offsets
// [128 P, 128 P + 32) from the 128-byte line below x, P < n_s) holds a key >= tau1.
// Chunks of the other sampled lines are not loaded: none of their elements can be
// admitted, so skipping them changes no result. The loads go through a buffer resource
// over the row's body: a skipped chunk is given an offset past the resource's end,
// which the hardware answers with zeros and no memory access. The loads stay
// unconditional in the control flow, so the compiler can still wait for one batch at
// a time. Without SKIP, lanes past the body's end read its last chunk again (always
// in bounds) and are masked.
// x[0, L) may be a segment of a row whose element 0 is row element ebase (candidates
// record row indices); with SKIP the segment must start on a sampled line, and P
// counts periods from there.
template <bool POS, bool SKIP>
__device__ __forceinline__ void fused_pass(grow_t x, uint32_t L, uint32_t n_s, const PassCtx c,
                                           uint32_t ebase = 0u) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  const uint32_t l = lane_id();
  uint32_t head = (uint32_t)((4u - ((uint32_t)((uintptr_t)x >> 2) & 3u)) & 3u);
  if (head > L) head = L;
  if (t < head) admit_one<POS>(true, x[t], ebase + t, c);
  const uint32_t nv = (L - head) >> 2;
  grow_t body = x + head;
  const uint32_t gb = ((uint32_t)((uintptr_t)x & 127u) >> 2) + head;  // body offset from the line below x
  constexpr uint32_t PERW = WAVE * PASS_UNROLL;  // quads per wave batch
  static_assert(4 * PERW / 128 + 1 + 31 < 64, "a batch's periods lie within two bitmap words");
  const uint32_t nb = (nv + PERW - 1u) / PERW;
  // Raw buffer over the body (16 nv bytes; rows with SKIP are at most 8192 sample
  // periods long). Word 3 is the gfx9-family buffer format word; the load's cache
  // policy 2 is "nt".
  // The base and size are the same in every lane; reading them from the first lane
  // puts the resource in scalar registers (otherwise each load is wrapped in a loop
  // over the distinct resource values).
  const uint64_t bp = (uint64_t)(uintptr_t)body;
  const uint32_t bp_lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bp);
  const uint32_t bp_hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(bp >> 32));
  const int nrec = __builtin_amdgcn_readfirstlane(SKIP ? (int)(16u * nv) : 0);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(uintptr_t)(((uint64_t)bp_hi << 32) | bp_lo), (short)0, nrec, 0x00020000);
  // Loads batch b; inert[u] receives the value to OR into chunk u before it is
  // examined (never_admitted for a skipped or past-the-end chunk, else 0). Applying it
  // at examination rather than here keeps the compiler from waiting for the prefetched
  // batch, and keeps the loads themselves unconditional (no branch around them). The
  // batch's periods lie within two bitmap words, read once per batch.
  auto fetch = [&](uint32_t b, u32x4 (&v)[PASS_UNROLL], uint32_t (&inert)[PASS_UNROLL]) {
    const uint32_t q0 = b * PERW;
    uint64_t hot = 0;
    uint32_t p0 = 0;
    if (SKIP) {
      const uint32_t w0 = (gb + 4u * q0) >> 12;  // bitmap word of the batch's first period
      hot = (uint64_t)s.fl_idx[w0 & (uint32_t)(FL_CAP - 1)] |
            ((uint64_t)s.fl_idx[(w0 + 1u) & (uint32_t)(FL_CAP - 1)] << 32);
      p0 = 32u * w0;
    }
#pragma unroll
    for (int u = 0; u < PASS_UNROLL; ++u) {
      const uint32_t q = q0 + (uint32_t)u * WAVE + l;
      const bool past = q >= nv;
      if (SKIP) {
        const uint32_t g = gb + 4u * q;
        const uint32_t P = g >> 7;
        const bool cold = ((g >> 5) & 3u) == 0u && P < n_s && ((hot >> (P - p0)) & 1u) == 0u;
        const bool off = past | cold;
        inert[u] = off ? never_admitted<POS>() : 0u;
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off ? 0xFFFFFFF0u : 16u * q, 0, 2);
      } else {
        inert[u] = past ? never_admitted<POS>() : 0u;
        v[u] = load4_stream(body + 4u * (past ? nv - 1u : q));
      }
    }
  };
  auto claim = [&]() -> uint32_t {
    uint32_t v = 0;
    if (l == 0) v = atomicAdd(&s.pass_next, 1u);
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
  };
  // Masking is needed only where a chunk that must not be admitted can read as an
  // admitted value: without SKIP, in the last batch (its chunks past the end re-read the
  // body's last chunk); with SKIP, where zeros (what a skipped chunk reads) are admitted,
  // i.e. unless the admission threshold is above +0.
  const bool skip_masked = !(POS && c.thr != 0u);
  auto examine = [&](const u32x4 (&raw)[PASS_UNROLL], const uint32_t (&inert)[PASS_UNROLL], uint32_t b) {
    u32x4 v[PASS_UNROLL];
    uint32_t e[PASS_UNROLL];
#pragma unroll
    for (int u = 0; u < PASS_UNROLL; ++u) {
      v[u] = raw[u];
      e[u] = ebase + head + 4u * (b * PERW + (uint32_t)u * WAVE + l);
    }
    if (SKIP ? skip_masked : (b + 1u == nb)) {
#pragma unroll
      for (int u = 0; u < PASS_UNROLL; ++u) v[u] = v[u] | splat4(inert[u]);
    }
    admit_batch<POS, PASS_UNROLL>(v, e, c);
  };
  uint32_t b = claim();
  if (b < nb) {
    u32x4 a[PASS_UNROLL];
    uint32_t am[PASS_UNROLL];
    fetch(b, a, am);
    for (;;) {
      const uint32_t bn = claim();
      if (bn >= nb) {
        examine(a, am, b);
        break;
      }
      u32x4 nx[PASS_UNROLL];
      uint32_t nm[PASS_UNROLL];
      fetch(bn, nx, nm);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the examination
      examine(a, am, b);
#pragma unroll
      for (int u = 0; u < PASS_UNROLL; ++u) {
        a[u] = nx[u];
        am[u] = nm[u];
      }
      b = bn;
    }
  }
  const uint32_t tail0 = head + 4u * nv;
  if (t < L - tail0) admit_one<POS>(true, x[tail0 + t], ebase + tail0 + t, c);
}

// After a pass that admitted n <= CAP keys: the admitted keys >= k0 and >= k1, read
// from the list in LDS, in s.cnt0 and s.cnt1 (zeroed by reset_row_state). Counting
// here rather than in the pass keeps two instructions per examined slot out of the
// pass, which is short of vector ALU time on rows of 128K. Ends with a barrier.
__device__ __forceinline__ void count_admitted(uint32_t n, uint32_t k0, uint32_t k1) {
  Smem& s = g_s;
  // Both counts in one word (each at most CAP per wave), summed over the wave.
  uint32_t ab = 0;
  for (uint32_t i = threadIdx.x; i < n; i += BLOCK) {
    const uint32_t k = s.buf[CAP + i];
    ab += (k >= k0 ? 1u : 0u) + (k >= k1 ? 0x10000u : 0u);
  }
  ab = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(ab), WAVE - 1);
  if (lane_id() == 0 && ab != 0) {
    atomicAdd(&s.cnt0, ab & 0xFFFFu);
    atomicAdd(&s.cnt1, ab >> 16);
  }
  __syncthreads();
}

// ------------------------------------------------ line-granular sampling
//
// HBM moves whole 128-byte lines, so the 4-byte read of x[j*128] costs a full line
// (a quarter of the row's bytes at stride 128). The sampler therefore reads each
// sampled line whole: the element at j*128 is still the sample key (the proposal
// is unchanged), and the line's maximum key is kept alongside it. The full-row pass
// then skips every sampled line whose maximum is below tau1 (no element of it can be
// admitted) and reads the "hot" ones again. It pays where few sampled lines are hot
// (tau1 deep in the tail of long rows); the host enables it by shape.
//
// Geometry: offsets are counted in floats from base = x rounded down to a 128-byte
// line, so element index = offset - off4 with off4 = (x & 127) / 4. The line of
// x[j*128] starts at offset 128 j (adding 512 j bytes keeps the low seven address
// bits). Period p = offsets [128 p, 128 p + 128): its first line is sampled when
// p < n_s and its other three lines are not. Past period n_s - 1 the row can reach
// only into the first line of period n_s, which is not sampled.

constexpr uint32_t LINE_SAMPLE_MAX = 8192;              // n_s limit of line sampling
constexpr int LM_PER_THREAD = LINE_SAMPLE_MAX / BLOCK;  // sampled lines per thread
static_assert(LINE_SAMPLE_MAX / 32 <= FL_CAP, "the hot-line bitmap lives in the frontier index list");
static_assert(BLOCK % 64 == 0 && LINE_SAMPLE_MAX % BLOCK == 0, "bitmap words are written per wave");
constexpr int SAMPLE_UNROLL = 6;

// Reads the sampled lines j0 <= j < j1 whole. skey[j] = key(x[j*128]); lmax[j] = max
// key of the line's elements inside the row; mn/mx fold this thread's sample keys.
// Eight lanes read one line (one 16-byte chunk each); batches of SAMPLE_UNROLL
// loads per lane are double-buffered so the next batch is in flight while the
// current one is reduced. P is an LDS or a global pointer type.
template <bool STREAM = false, class P>
__device__ __forceinline__ void sample_lines_range(grow_t x, uint32_t L, uint32_t j0, uint32_t j1, P skey,
                                                   P lmax, uint32_t& mn, uint32_t& mx) {
  const uint32_t t = threadIdx.x;
  const uint32_t off4 = (uint32_t)((uintptr_t)x & 127u) >> 2;
  grow_t base = x - off4;
  const uint32_t c = t & 7;          // this lane's 16-byte chunk of the line
  const uint32_t cs = off4 >> 2;     // chunk holding x[j*128]
  const uint32_t is = off4 & 3u;     // component holding x[j*128]
  const uint32_t lo = off4, hi = off4 + L;  // valid offsets [lo, hi)
  const uint32_t gfirst = off4 & ~3u;        // chunk holding the row's first element
  const uint32_t glast = (hi - 1u) & ~3u;    // chunk holding the row's last element
  constexpr uint32_t LINES_PER_STEP = BLOCK / 8;
  constexpr uint32_t STEP = LINES_PER_STEP * SAMPLE_UNROLL;  // lines per batch
  // Chunks outside the row read the row's first or last chunk instead (always in
  // bounds, unconditional); their elements are masked out when reduced.
  auto fetch = [&](u32x4 (&v)[SAMPLE_UNROLL], uint32_t step) {
#pragma unroll
    for (int u = 0; u < SAMPLE_UNROLL; ++u) {
      const uint32_t j = j0 + step * STEP + u * LINES_PER_STEP + (t >> 3);
      const uint32_t g = 128u * j + 4u * c;
      const grow_t a = base + (g < gfirst ? gfirst : (g < glast ? g : glast));
      v[u] = STREAM ? load4_stream(a) : load4(a);
    }
  };
  auto reduce = [&](const u32x4 (&v)[SAMPLE_UNROLL], uint32_t step) {
#pragma unroll
    for (int u = 0; u < SAMPLE_UNROLL; ++u) {
      const uint32_t j = j0 + step * STEP + u * LINES_PER_STEP + (t >> 3);
      const uint32_t g = 128u * j + 4u * c;
      uint32_t m = 0;
      if (j < j1 && g + 0 >= lo && g + 0 < hi) m = max(m, key_of_bits(v[u].x));
      if (j < j1 && g + 1 >= lo && g + 1 < hi) m = max(m, key_of_bits(v[u].y));
      if (j < j1 && g + 2 >= lo && g + 2 < hi) m = max(m, key_of_bits(v[u].z));
      if (j < j1 && g + 3 >= lo && g + 3 < hi) m = max(m, key_of_bits(v[u].w));
      // Maximum over the line's eight lanes: within each quad, then the two quads of
      // the eight-lane group exchange through row shifts by 4 limited to their banks.
      m = max(m, dpp<DPP_QUAD_SWAP1>(0u, m));
      m = max(m, dpp<DPP_QUAD_SWAP2>(0u, m));
      m = max(m, dpp<DPP_ROW_SHR + 4, 0xf, 0xa>(0u, m));
      m = max(m, dpp<DPP_ROW_SHL + 4, 0xf, 0x5>(0u, m));
      if (j < j1) {
        if (c == 0) lmax[j] = m;
        if (c == cs) {
          const uint32_t w = is == 0 ? v[u].x : is == 1 ? v[u].y : is == 2 ? v[u].z : v[u].w;
          const uint32_t k = key_of_bits(w);
          skey[j] = k;
          mn = min(mn, k);
          mx = max(mx, k);
        }
      }
    }
  };
  const uint32_t nsteps = (j1 - j0 + STEP - 1) / STEP;
  if (nsteps == 0) return;
  u32x4 a[SAMPLE_UNROLL], b[SAMPLE_UNROLL];
  fetch(a, 0);
  uint32_t i = 0;
  for (; i + 2 < nsteps; i += 2) {
    fetch(b, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    reduce(a, i);
    fetch(a, i + 2);
    __builtin_amdgcn_sched_barrier(0);
    reduce(b, i + 1);
  }
  if (i + 1 < nsteps) {
    fetch(b, i + 1);
    __builtin_amdgcn_sched_barrier(0);
    reduce(a, i);
    reduce(b, i + 1);
  } else {
    reduce(a, i);
  }
}

// The whole row's sample into LDS, with the min/max sample key in s.mn/s.mx.
template <bool STREAM>
__device__ __forceinline__ void sample_lines(grow_t x, uint32_t L, uint32_t n_s, uint32_t* skey, uint32_t* lmax) {
  uint32_t mn = KEY_MAX, mx = 0;
  sample_lines_range<STREAM>(x, L, 0u, n_s, skey, lmax, mn, mx);
  block_minmax(mn, mx);
}

// Boundary refinement and commit of an LDS list of n keys whose first histogram,
// over (key - base) >> sh (top bin clamped), is in s.hist, with the row counters
// zeroed: the bins above the bin holding rank K are committed in one pass, that
// bin's keys move to the frontier buffer (or, when too many, only their extremes are
// noted), and the frontier is resolved exactly.
//
// With COUNT, the first sweep also counts the listed keys >= k0 and >= k1 into s.cnt0
// and s.cnt1 (zeroed by reset_row_state), which hold the totals once this returns.
template <bool KEYS_ONLY, bool COUNT>
__device__ __forceinline__ void refine_list(uint32_t n, uint32_t K, uint32_t base, uint32_t sh, RowOut out,
                                            Control* ctl, uint32_t k0, uint32_t k1) {
  Smem& s = g_s;
  // The list: (index, key) pairs at s.buf[i], s.buf[CAP + i], or keys only at s.buf[i]
  // with the position as the index.
  auto key_at = [&](uint32_t i) -> uint32_t { return KEYS_ONLY ? g_s.buf[i] : g_s.buf[CAP + i]; };
  // Entries i .. i + 3 (i a multiple of 4 below n; the reads stay inside the list's region,
  // entries at n and beyond are stale and masked by the callers).
  auto keys4_at = [&](uint32_t i) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(KEYS_ONLY ? &g_s.buf[i] : &g_s.buf[CAP + i]);
  };
  auto ids4_at = [&](uint32_t i) -> u32x4 {
    if (KEYS_ONLY) return u32x4{i, i + 1u, i + 2u, i + 3u};
    return *reinterpret_cast<const u32x4*>(&g_s.buf[i]);
  };
  if (threadIdx.x == 0) {  // extremes of the boundary bin's keys (block_find_bin's barrier orders this)
    s.mn = KEY_MAX;
    s.mx = 0;
  }
  block_find_bin(K);
  const uint32_t b = s.sel_bin, above = s.sel_above;
  const uint32_t cb = s.hist[b];
  const uint32_t need = K - above;
  const uint32_t blo = base + (b << sh);
  const uint32_t wdt = (1u << sh) - 1u;
  const uint32_t bhi = (b == (uint32_t)(NB - 1)) ? KEY_MAX
                                                 : blo + ((KEY_MAX - blo) < wdt ? (KEY_MAX - blo) : wdt);
  const bool fits = cb <= (uint32_t)FL_CAP;
  // Commit the resolved bins above b; move bin b to the frontier buffer, or, when it
  // is too wide for it, note the extremes of its keys.
  // Two sweeps over the list: count this thread's keys above the bin and in it (and
  // note the bin's extremes), reserve their slots once per wave, then write them.
  // Each thread takes four consecutive entries per step (16-byte LDS reads, several in
  // flight), so the sweeps wait on one LDS round trip per four entries.
  uint32_t bmn = KEY_MAX, bmx = 0, ng = 0, nin = 0, cnt01 = 0;
  for (uint32_t i = 4u * threadIdx.x; i < n; i += 4u * BLOCK) {
    const u32x4 k4 = keys4_at(i);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t k = k4[u];
      const bool v = i + (uint32_t)u < n;
      const bool in = v && k >= blo && k <= bhi;
      ng += (v && k > bhi) ? 1u : 0u;
      nin += in ? 1u : 0u;
      if (COUNT) cnt01 += v ? (k >= k0 ? 1u : 0u) + (k >= k1 ? 0x10000u : 0u) : 0u;
      bmn = in ? min(bmn, k) : bmn;
      bmx = in ? max(bmx, k) : bmx;
    }
  }
  {
    uint32_t p = wave_reserve_n<LIST_BITS>(ng, &s.out_gt);
    uint32_t f = fits ? wave_reserve_n<LIST_BITS>(nin, &s.fl_cnt) : 0u;
    if (ng + (fits ? nin : 0u) != 0) {
      for (uint32_t i = 4u * threadIdx.x; i < n; i += 4u * BLOCK) {
        const u32x4 k4 = keys4_at(i);
        const u32x4 id4 = ids4_at(i);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t k = k4[u];
          const bool v = i + (uint32_t)u < n;
          const bool g = v && k > bhi;
          const bool in = v && fits && !g && k >= blo;
          if (g && p < K) out.put(p, id4[u], k);
          if (in && f < (uint32_t)FL_CAP) {
            s.fl_idx[f] = id4[u];
            s.fl_key[f] = k;
          }
          p += g ? 1u : 0u;
          f += in ? 1u : 0u;
        }
      }
    }
  }
  bmn = wave_min_u32(bmn);
  bmx = wave_max_u32(bmx);
  if (COUNT) cnt01 = (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(cnt01), WAVE - 1);
  if (lane_id() == 0) {
    atomicMin(&s.mn, bmn);
    atomicMax(&s.mx, bmx);
    if (COUNT && cnt01 != 0u) {
      atomicAdd(&s.cnt0, cnt01 & 0xFFFFu);
      atomicAdd(&s.cnt1, cnt01 >> 16);
    }
  }
  __syncthreads();
  uint32_t T, gt2;
  if (fits && cb <= FL_RANK_MAX) {
    // A short frontier: each thread ranks one of its keys, and the first `need` in
    // (key descending, position ascending) order are committed.
    const uint32_t rk = rank_in_list(s.fl_key, cb);
    const bool sel = rk < need;
    const uint32_t pp = wave_reserve(sel, &s.out_gt);
    if (sel && pp < K) out.put(pp, s.fl_idx[threadIdx.x], s.fl_key[threadIdx.x]);
  } else if (fits) {
    // A longer frontier (one key per thread): find the K-th key T inside it, from the
    // extremes when it is a single repeated key, else by radix narrowing over
    // [min, max]; commit the keys above T and `need - gt` of the copies of T (ties at
    // the boundary may go either way).
    const uint32_t mn = s.mn, mx = s.mx;
    if (mn == mx) {
      T = mn;
      gt2 = 0;
    } else {
      select_rank([&](auto&& f) {
        if (threadIdx.x < cb) f(g_s.fl_key[threadIdx.x]);
      }, need, mn, mx, T, gt2);
    }
    const uint32_t gt_total = above + gt2;
    const uint32_t ties = K - gt_total;
    const bool has = threadIdx.x < cb;
    const uint32_t k = has ? s.fl_key[threadIdx.x] : 0u;
    const uint32_t id = has ? s.fl_idx[threadIdx.x] : 0u;
    const bool g = has && k > T;
    const uint32_t pg = wave_reserve(g, &s.out_gt);
    if (g && pg < K) out.put(pg, id, k);
    const bool e = has && k == T;
    const uint32_t q = wave_reserve(e, &s.out_tie);
    if (e && q < ties && gt_total + q < K) out.put(gt_total + q, id, k);
  } else {
    if (threadIdx.x == 0) stat_add(ctl, TOPK_STAT_FRONTIER_WIDE);
    if (s.mn == s.mx) {
      // The whole boundary bin is one repeated key (typical of bf16-rounded scores):
      // it is the K-th key, and `need` of its copies complete the output.
      T = s.mn;
      gt2 = 0;
    } else {
      select_rank([&](auto&& f) {
        for (uint32_t i = threadIdx.x; i < n; i += BLOCK) f(key_at(i));
      }, need, blo, bhi, T, gt2);
    }
    const uint32_t gt_total = above + gt2;
    const uint32_t ties = K - gt_total;
    uint32_t ng = 0, ne = 0;
    for (uint32_t i = 4u * threadIdx.x; i < n; i += 4u * BLOCK) {
      const u32x4 k4 = keys4_at(i);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t k = k4[u];
        const bool v = i + (uint32_t)u < n;
        ng += (v && k > T && k <= bhi) ? 1u : 0u;
        ne += (v && k == T) ? 1u : 0u;
      }
    }
    uint32_t p = wave_reserve_n<LIST_BITS>(ng, &s.out_gt);
    uint32_t q = wave_reserve_n<LIST_BITS>(ne, &s.out_tie);
    if (ng + ne != 0) {
      for (uint32_t i = 4u * threadIdx.x; i < n; i += 4u * BLOCK) {
        const u32x4 k4 = keys4_at(i);
        const u32x4 id4 = ids4_at(i);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t k = k4[u];
          const bool v = i + (uint32_t)u < n;
          const bool g = v && k > T && k <= bhi;
          const bool e = v && k == T;
          if (g && p < K) out.put(p, id4[u], k);
          if (e && q < ties && gt_total + q < K) out.put(gt_total + q, id4[u], k);
          p += g ? 1u : 0u;
          q += e ? 1u : 0u;
        }
      }
    }
  }
}

// After a certified sampled pass: n = C(tau1) <= CAP candidates in LDS with the first
// histogram over (key - key(tau1)) >> sh.
__device__ __forceinline__ void refine_commit(uint32_t n, uint32_t K, const PassCtx c, RowOut out, Control* ctl) {
  refine_list<false>(n, K, c.akey, c.sh, out, ctl);
}

__device__ __forceinline__ PassCtx pass_ctx(uint32_t akey, uint32_t smax) {
  PassCtx c;
  c.akey = akey;
  c.sh = shift_for(smax - akey);
  c.thr = akey >= 0x80000000u ? (akey ^ 0x80000000u) : ~akey;
  return c;
}

// Exact recovery of a row by its own workgroup: one more pass over the row admitting
// keys >= thr (a threshold below the K-th key: the deeper sample rank for an
// underfilled row, the boundary bin of the pass histogram for an overflowing one);
// when its count certifies (K <= C(thr) <= CAP) the admitted list is refined as usual,
// otherwise (or with thr = 0) the exact full-row select over [lo, hi] runs. Nothing has
// been written to the row's output yet. Out of line: the path is rare, and inlined its
// second pass would raise the register pressure of every kernel that holds it.
// Takes scalars only: a reference to the launch parameters would force them into
// scratch memory in every caller.
__device__ __attribute__((noinline)) void recover_in_place(grow_t x, uint32_t L, uint32_t K, uint32_t thr,
                                                           uint32_t smax, uint32_t lo, uint32_t hi, RowOut out,
                                                           Control* ctl) {
  Smem& s = g_s;
  if (threadIdx.x == 0) stat_add(ctl, TOPK_STAT_RECOVER_INPLACE);
  if (thr != 0u) {
    reset_row_state();
    const PassCtx c = pass_ctx(thr, smax > thr ? smax : thr);
    if (thr >= 0x80000000u) fused_pass<true, false>(x, L, 0u, c);
    else fused_pass<false, false>(x, L, 0u, c);
    __syncthreads();
    const uint32_t n = s.cnt;
    if (n >= K && n <= (uint32_t)CAP) {
      if (threadIdx.x == 0) stat_add(ctl, TOPK_STAT_INPLACE_CERTIFIED);
      refine_commit(n, K, c, out, ctl);
      return;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) stat_add(ctl, TOPK_STAT_INPLACE_FULL);
  exact_full_row(x, L, K, lo, hi, out, ctl);
}

// For a row whose admitted keys overflowed the buffer (C(tau1) > CAP >= K): the pass
// histogram s.hist over (key - t1key) >> sh counted every admitted key, so the bin
// holding rank K is known; returns its lowest key, with n_ge = the keys at or above it.
__device__ __forceinline__ uint32_t overflow_threshold(uint32_t K, uint32_t t1key, uint32_t sh, uint32_t& n_ge) {
  block_find_bin(K);
  const uint32_t b = g_s.sel_bin;
  n_ge = g_s.sel_above + g_s.hist[b];
  __syncthreads();
  return t1key + (b << sh);
}

// Hands a row whose K-th key lies in [wlo, whi] to the collect and finish recovery
// kernels (no histogram pass): `above` keys of the row exceed whi; with commit they are
// committed by the collect kernel, otherwise the caller has already written them to
// output slots [0, above). If the queue is full the row is recovered here instead (the
// exact full-row select over [lo, hi], which rewrites every slot).
__device__ __forceinline__ void recover_row_window(const Params& p, uint32_t row, grow_t x, uint32_t L, uint32_t wlo,
                                                   uint32_t whi, uint32_t above, bool commit, uint32_t lo,
                                                   uint32_t hi, RowOut out) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  if (t == 0) s.bcast = atomicAdd(&p.ctl->qcount, 1u);
  __syncthreads();
  const uint32_t q = s.bcast;
  __syncthreads();
  if (q < p.qmax) {
    if (t == 0) {
      s.queued = 1u;
      RecSlot* r = p.rec + q;
      r->row = row;
      r->L = L;
      r->lo = lo;
      r->hi = hi;
      r->mode = REC_WINDOW;
      r->commit = commit ? 1u : 0u;
      r->bin_lo = wlo;
      r->bin_hi = whi;
      r->bin_above = above;
      r->out_gt = commit ? 0u : above;
      r->cnt = 0;
      stat_add(p.ctl, TOPK_STAT_QUEUED);
    }
  } else {
    if (t == 0) {
      stat_add(p.ctl, TOPK_STAT_RECOVER_INPLACE);
      stat_add(p.ctl, TOPK_STAT_INPLACE_FULL);
    }
    exact_full_row(x, L, p.K, lo, hi, out, p.ctl);
  }
}

// An overflowing row (C(tau1) > CAP >= K) for the recovery kernels: the pass histogram
// s.hist over (key - t1key) >> sh counted every admitted key, so the bin holding rank K
// and the count of keys above it are known, and the collect kernel commits the keys
// above that bin and gathers the bin itself.
__device__ __forceinline__ void queue_overflow(const Params& p, uint32_t row, grow_t x, uint32_t L, uint32_t t1key,
                                               uint32_t sh, uint32_t smax, RowOut out) {
  block_find_bin(p.K);
  const uint32_t b = g_s.sel_bin, above = g_s.sel_above;
  const uint32_t blo = t1key + (b << sh);
  const uint32_t wdt = (1u << sh) - 1u;
  const uint32_t bhi = (b == (uint32_t)(NB - 1)) ? KEY_MAX : blo + ((KEY_MAX - blo) < wdt ? (KEY_MAX - blo) : wdt);
  recover_row_window(p, row, x, L, blo, bhi, above, true, t1key, smax, out);
}

// An underfilled row (C(tau1) < K) for the recovery kernels: its C(tau1) admitted keys
// (idx[i], key[i], i < c1) are all in the top K and are committed here; the remaining
// K - C(tau1) lie below tau1, and the collect kernel gathers [tau2, tau1) for them. If
// that window holds too few, the finish kernel selects over the whole row instead.
template <class P>
__device__ __forceinline__ void queue_underfill(const Params& p, uint32_t row, grow_t x, uint32_t L, uint32_t c1,
                                                uint32_t t1key, uint32_t t2key, uint32_t smin, P idx, P key,
                                                RowOut out) {
  for (uint32_t i = threadIdx.x; i < c1; i += BLOCK) out.put(i, idx[i], key[i]);
  recover_row_window(p, row, x, L, t2key, t1key - 1u, c1, false, smin, t1key, out);
}

// Hands a row that needs exact full-row recovery to the cooperative recovery
// kernels (which run after this kernel and spread the row over the whole GPU), or
// recovers it here when the queue is full. Nothing has been written to the row's
// output yet. [lo, hi] is the key range the recovery histogram bins.
__device__ __forceinline__ void recover_row(const Params& p, uint32_t row, grow_t x, uint32_t L, uint32_t lo, uint32_t hi,
                            RowOut out) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  if (t == 0) s.bcast = atomicAdd(&p.ctl->qcount, 1u);
  __syncthreads();
  const uint32_t q = s.bcast;
  __syncthreads();
  if (q < p.qmax) {
    RecSlot* r = p.rec + q;
    if (t == 0) {
      s.queued = 1u;
      r->row = row;
      r->L = L;
      r->lo = lo;
      r->hi = hi;
      r->mode = REC_HIST;
      r->commit = 1u;
      r->out_gt = 0;
      r->cnt = 0;
      stat_add(p.ctl, TOPK_STAT_QUEUED);
    }
    for (uint32_t i = t; i < (uint32_t)NB; i += BLOCK) r->hist[i] = 0;
  } else {
    if (t == 0) {
      stat_add(p.ctl, TOPK_STAT_RECOVER_INPLACE);
      stat_add(p.ctl, TOPK_STAT_INPLACE_FULL);
    }
    exact_full_row(x, L, p.K, lo, hi, out, p.ctl);
  }
}

// tau1, tau0, taua and tau2: the r1-th, r0-th, ra-th and r2-th largest
// (r0 <= r1 <= ra <= r2) of the n_s sample keys in s.buf[0, n_s), all inside [mn, mx].
// One radix round finds the bin holding rank r2; when the keys in that bin and above fit
// the frontier buffer (the usual case, r2 is a few dozen), the four ranks are read off by
// counting inside that short list. Otherwise the general narrowing selection runs.
__device__ __forceinline__ void select_taus(uint32_t n_s, uint32_t r0, uint32_t r1, uint32_t ra, uint32_t r2,
                                            uint32_t mn, uint32_t mx, uint32_t& t0key, uint32_t& t1key,
                                            uint32_t& takey, uint32_t& t2key, bool hist_is_zero = false) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  const uint32_t sh = shift_for(mx - mn);
  if (!hist_is_zero) {
    for (uint32_t i = t; i < (uint32_t)NB; i += BLOCK) s.hist[i] = 0;
    if (t == 0) s.fl_cnt = 0;
    __syncthreads();
  }
  // Four sample keys per 16-byte LDS read; entries from n_s on are stale and skipped.
  for (uint32_t i = 4u * t; i < n_s; i += 4u * BLOCK) {
    const u32x4 k4 = *reinterpret_cast<const u32x4*>(&s.buf[i]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + (uint32_t)u < n_s) atomicAdd(&s.hist[(k4[u] - mn) >> sh], 1u);
  }
  __syncthreads();
  block_find_bin(r2);
  const uint32_t b = s.sel_bin;
  const uint32_t m = s.sel_above + s.hist[b];  // sample keys in bin b and above
  const uint32_t blo = mn + (b << sh);
  if (m <= (uint32_t)FL_CAP) {
    uint32_t nin = 0;
    for (uint32_t i = 4u * t; i < n_s; i += 4u * BLOCK) {
      const u32x4 k4 = *reinterpret_cast<const u32x4*>(&s.buf[i]);
#pragma unroll
      for (int u = 0; u < 4; ++u) nin += (i + (uint32_t)u < n_s && k4[u] >= blo) ? 1u : 0u;
    }
    uint32_t f = wave_reserve_n<LIST_BITS>(nin, &s.fl_cnt);
    if (nin != 0) {
      for (uint32_t i = 4u * t; i < n_s; i += 4u * BLOCK) {
        const u32x4 k4 = *reinterpret_cast<const u32x4*>(&s.buf[i]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool in = i + (uint32_t)u < n_s && k4[u] >= blo;
          if (in && f < (uint32_t)FL_CAP) s.fl_key[f] = k4[u];
          f += in ? 1u : 0u;
        }
      }
    }
    __syncthreads();
    if (m <= (uint32_t)WAVE) {
      // Every wave sorts the short list across its lanes and reads the three ranks off:
      // no rank counting by one wave, no barrier to broadcast the result. (The list is
      // not written again before the next row's barriers.)
      const uint32_t l = lane_id();
      const uint32_t srt = wave_sort_desc(l < m ? s.fl_key[l] : 0u);
      t1key = (uint32_t)__builtin_amdgcn_readlane((int)srt, (int)(r1 - 1));
      t0key = (uint32_t)__builtin_amdgcn_readlane((int)srt, (int)(r0 - 1));
      takey = (uint32_t)__builtin_amdgcn_readlane((int)srt, (int)(ra - 1));
      t2key = (uint32_t)__builtin_amdgcn_readlane((int)srt, (int)(r2 - 1));
    } else {
      const uint32_t rk = rank_in_list(s.fl_key, m);
      if (rk == r1 - 1) s.sel_above = s.fl_key[t];
      if (rk == r0 - 1) s.sel_bin = s.fl_key[t];
      if (rk == ra - 1) s.bcast2 = s.fl_key[t];
      if (rk == r2 - 1) s.bcast = s.fl_key[t];
      __syncthreads();
      t1key = s.sel_above;
      t0key = s.sel_bin;
      takey = s.bcast2;
      t2key = s.bcast;
      __syncthreads();
    }
  } else {
    uint32_t unused;
    select_rank([&](auto&& f) {
      for (uint32_t i = threadIdx.x; i < n_s; i += BLOCK) f(g_s.buf[i]);
    }, r2, mn, mx, t2key, unused);
    select_rank([&](auto&& f) {
      for (uint32_t i = threadIdx.x; i < n_s; i += BLOCK) f(g_s.buf[i]);
    }, r1, t2key, mx, t1key, unused);
    select_rank([&](auto&& f) {
      for (uint32_t i = threadIdx.x; i < n_s; i += BLOCK) f(g_s.buf[i]);
    }, r0, t1key, mx, t0key, unused);
    takey = t1key;
    if (ra != r1) {
      select_rank([&](auto&& f) {
        for (uint32_t i = threadIdx.x; i < n_s; i += BLOCK) f(g_s.buf[i]);
      }, ra, t2key, mx, takey, unused);
    }
  }
}

__device__ __forceinline__ uint32_t sample_rank(uint32_t target, uint32_t n_s, uint32_t L) {
  uint64_t r = ((uint64_t)target * n_s + L - 1) / L;
  if (r < 1) r = 1;
  if (r > n_s) r = n_s;
  return (uint32_t)r;
}

// Bitmap of the hot sampled lines (line maximum lmax[j] >= tau1 key) in s.fl_idx, which
// the frontier uses only after the pass: bit j of the list, j < n_s. Each wave writes the
// two words of its 64 lines per step through one base address and constant offsets, so
// no per-step address stays live across the row loop.
__device__ __forceinline__ void write_hot_bitmap(const uint32_t* lmax, uint32_t n_s, uint32_t t1key) {
  const uint32_t t = threadIdx.x;
  const uint32_t* lm = lmax + t;
  uint32_t* words = &g_s.fl_idx[2u * (t / WAVE) + (lane_id() & 1u)];
  const uint32_t nj = n_s - t;  // lines j = t + m BLOCK below n_s: m BLOCK < nj
#pragma unroll
  for (int m = 0; m < LM_PER_THREAD; ++m) {
    const uint64_t hb = __ballot((uint32_t)m * BLOCK < nj && n_s > t && lm[m * BLOCK] >= t1key);
    if (lane_id() < 2) words[m * (BLOCK / 32)] = (lane_id() & 1u) ? (uint32_t)(hb >> 32) : (uint32_t)hb;
  }
}

template <bool STREAM_SAMPLE>
__device__ __forceinline__ void sampled_row(const Params& p, uint32_t row, grow_t x, uint32_t L, RowOut out) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  // Rows whose stride-s sample would not fit the LDS key list (L > 16384 s, past the
  // widths the method is defined on) keep a fixed stride, doubled until it fits: the
  // positions stay on the stride-s grid, and the proposal only steers the work.
  uint32_t stride = p.stride;
  while ((L + stride - 1) / stride > (uint32_t)KEYS_CAP) stride *= 2u;
  const uint32_t n_s = (L + stride - 1) / stride;
  if (t == 0) {
    stat_add(p.ctl, TOPK_STAT_SAMPLED);
    if (stride != p.stride) stat_add(p.ctl, TOPK_STAT_LONG_EXACT);
  }
  // Fixed-stride row-local view: keys of x[j * s], j < ceil(L / s), in s.buf[0, n_s).
  // Line-granular sampling (and the line skipping it enables) holds at the method's
  // stride of 128 and is used where it pays (p.line_min, chosen by shape on the host);
  // otherwise, and for other strides, the sample is read element by element and the
  // full pass reads the whole row.
  const bool by_lines = stride == STRIDE && n_s <= LINE_SAMPLE_MAX && n_s >= p.line_min;
  if (by_lines) {
    sample_lines<STREAM_SAMPLE>(x, L, n_s, &s.buf[0], &s.buf[CAP]);
  } else {
    uint32_t mn = KEY_MAX, mx = 0;
#pragma unroll 8
    for (uint32_t jr = t; jr < n_s; jr += BLOCK) {
      // Last sample first: the lines read last are the ones the pass, which runs
      // from the row's start, meets first, while they are still cached.
      const uint32_t j = n_s - 1u - jr;
      const uint32_t k = key_of_bits(x[(size_t)j * stride]);
      s.buf[j] = k;
      mn = min(mn, k);
      mx = max(mx, k);
    }
    block_minmax(mn, mx);
  }
  const uint32_t smin = s.mn, smax = s.mx;
  phase_mark(p.phase, row, PH_SAMPLED);
  const uint32_t r1 = sample_rank(p.T1, n_s, L);
  const uint32_t r0 = sample_rank(p.T0, n_s, L);
  const uint32_t r2 = sample_rank(p.T2, n_s, L);
  // Rows sampled one element per period admit keys down to the deeper sample rank ra
  // (target T_A): their C(tau1) spreads by about 1/sqrt(r1) around T1 and falls short of
  // K in a few rows per thousand, each of which would need one more read of the row,
  // while C(tau_a) almost never falls short of K or exceeds the buffer. C(tau0) and
  // C(tau1) are then counted among the admitted keys, so each row still reports the
  // threshold that certifies it. Line-sampled rows (32 keys per period, a far narrower
  // spread) admit at tau1, on which their line skipping is built.
  const uint32_t ra = by_lines ? r1 : sample_rank(p.TA, n_s, L);
  uint32_t t1key, t0key, takey, t2key;
  // The histogram and list counters are still zero from the row's reset (the sample does
  // not touch them).
  select_taus(n_s, r0, r1, ra, r2, smin, smax, t0key, t1key, takey, t2key, true);
  phase_mark(p.phase, row, PH_PROPOSED);

  const uint32_t akey = takey;  // tau1 when ra = r1
  const PassCtx c = pass_ctx(akey, smax);
  const bool pos = akey >= 0x80000000u;
  // Skipping sampled lines needs a value that is never admitted, which exists
  // unless the admission key is the lowest possible key.
  const bool skip = by_lines && akey != 0u;
  if (skip) write_hot_bitmap(&s.buf[CAP], n_s, akey);
  reset_row_state();  // its barrier also ends every read of the line maxima in LDS
  if (skip) {
    if (pos) fused_pass<true, true>(x, L, n_s, c);
    else fused_pass<false, true>(x, L, n_s, c);
  } else if (pos) {
    fused_pass<true, false>(x, L, n_s, c);
  } else {
    fused_pass<false, false>(x, L, n_s, c);
  }
  __syncthreads();
  const uint32_t n = s.cnt;
  phase_mark(p.phase, row, PH_PASSED);
  if (n > (uint32_t)CAP) {
    // Too many admitted to hold: the K-th key is >= the admission key, recover exactly.
    // A short row is recovered in place from the boundary bin of the pass histogram, a
    // long one by the cooperative recovery kernels.
    phase_put(p.phase, row, PH_COUNTS, (unsigned long long)n);
    if (t == 0) stat_add(p.ctl, TOPK_STAT_RECOVER_OVER);
    if (L <= p.inplace_max) {
      uint32_t n_ge;
      const uint32_t thr = overflow_threshold(p.K, akey, c.sh, n_ge);
      phase_mark(p.phase, row, PH_END);
      recover_in_place(x, L, p.K, n_ge <= (uint32_t)CAP ? thr : 0u, smax, akey, smax, out, p.ctl);
      phase_mark(p.phase, row, PH_RECOVERED);
      phase_path(p.phase, row, PATH_RECOVER_INPLACE);
    } else {
      queue_overflow(p, row, x, L, akey, c.sh, smax, out);
      phase_mark(p.phase, row, PH_END);
      phase_path(p.phase, row, PATH_RECOVER_QUEUED);
    }
  } else if (n < p.K) {
    // Even the admission threshold underfills: the K-th key is below it. A short row is
    // recovered in place from the deeper sample rank tau2, a long one cooperatively.
    phase_put(p.phase, row, PH_COUNTS, (unsigned long long)n);
    if (t == 0) stat_add(p.ctl, TOPK_STAT_RECOVER_UNDER);
    phase_mark(p.phase, row, PH_END);
    if (L <= p.inplace_max) {
      recover_in_place(x, L, p.K, t2key, smax, smin, akey, out, p.ctl);
      phase_mark(p.phase, row, PH_RECOVERED);
      phase_path(p.phase, row, PATH_RECOVER_INPLACE);
    } else {
      queue_underfill(p, row, x, L, n, akey, t2key, smin, (const uint32_t*)&s.buf[0], (const uint32_t*)&s.buf[CAP],
                      out);
      phase_path(p.phase, row, PATH_RECOVER_QUEUED);
    }
  } else {
    // Certified (K <= C(tau_a) <= CAP): refine, counting C(tau0) and C(tau1) among the
    // admitted keys on the way, which name the threshold that certifies the row.
    refine_list<false, true>(n, p.K, c.akey, c.sh, out, p.ctl, t0key, t1key);
    const uint32_t c0 = s.cnt0, c1 = s.cnt1;
    const uint32_t path = c0 >= p.K ? PATH_TAU0 : (c1 >= p.K ? PATH_TAU1 : PATH_TAUA);
    if (t == 0) {
      stat_add(p.ctl, path == PATH_TAU0 ? TOPK_STAT_TAU0 : (path == PATH_TAU1 ? TOPK_STAT_TAU1 : TOPK_STAT_TAUA));
    }
    phase_mark(p.phase, row, PH_END);
    phase_put(p.phase, row, PH_COUNTS, (unsigned long long)c1 | ((unsigned long long)c0 << 32));
    phase_path(p.phase, row, path);
  }
}

__device__ __forceinline__ uint32_t row_length(const Params& p, uint32_t row) {
  const int32_t len = p.row_len[row];
  uint32_t L = len < 0 ? 0u : (uint32_t)len;
  return L > p.N ? p.N : L;
}

// ------------------------------------------------------------ sorted output
//
// The sorted, value-returning output (an option beyond the pages' unordered contract):
// one workgroup per row orders the row's selected entries by (key descending, index
// ascending), then writes the indices and their scores; slots past the row's valid
// entries keep the sentinel and get -inf. Entries are 64-bit composites
// (key << 32 | ~index), never 0 for a valid entry (indices are below 2^31), so the zero
// padding sorts last. Thread t holds entries t*EPT .. t*EPT+EPT-1 of the P = EPT * BLOCK.
// Each wave first sorts its own EPT * WAVE entries with a bitonic network: every stage is
// a separate instantiation with its run length and exchange distance known at compile
// time, distances below EPT stay in registers and those up to 32 EPT go across the lanes
// of the wave (see lane_xor64), so no stage needs a barrier. The waves' runs are then
// merged pairwise through LDS (merge path, three levels for eight waves), one barrier per
// level.

// Exchange of a 64-bit value with lane ^ M. The network is bound by vector ALU issue, so
// only the one-instruction quad permutes (M = 1, 2) use DPP; M = 4, 8, 16 go through the
// LDS crossbar's swizzle (bit mode: lane ^ M within groups of 32) and M = 32 through a
// permute, both issued to the LDS pipe instead of the vector ALU.
template <int M>
__device__ __forceinline__ uint32_t lane_xor_lds(uint32_t v) {
  if constexpr (M <= 2) return lane_xor<M>(v);
  else if constexpr (M <= 16) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (M << 10) | 0x1F);
  else return (uint32_t)__shfl_xor((int)v, M);
}
template <int M>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t v) {
  const uint32_t lo = lane_xor_lds<M>((uint32_t)v), hi = lane_xor_lds<M>((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Stage (KB, J): runs of 2^KB entries, exchange distance J. An entry e meets e ^ J; the
// lower entry of the pair keeps the larger value where bit KB of e is clear.
template <int EPT, int KB, uint32_t J, bool ALL_DESC = false>
__device__ __forceinline__ void sort_stage(uint64_t (&v)[EPT], uint32_t t, uint64_t (*c)[EPT * BLOCK],
                                           int& buf) {
  constexpr uint32_t K = 1u << KB;
  if constexpr (J < (uint32_t)EPT) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      if (((uint32_t)q & J) == 0u) {
        const int r = q | (int)J;
        const bool desc = ALL_DESC || ((t * EPT + (uint32_t)q) & K) == 0u;
        const uint64_t x = v[q], y = v[r];
        // One compare: with x == y swapping changes nothing, so "y > x" may stand for
        // "x < y" and its negation for "x > y".
        const bool swap = (y > x) == desc;
        v[q] = swap ? y : x;
        v[r] = swap ? x : y;
      }
    }
  } else {
    constexpr uint32_t M = J / EPT;  // partner thread t ^ M, same register slot
    const bool lo = (t & M) == 0u;
    const bool desc = ALL_DESC || ((t * EPT) & K) == 0u;  // K >= J >= EPT: the same for every slot
    const bool keep_max = desc == lo;
    static_assert(M < (uint32_t)WAVE, "stages stay inside a wave");
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const uint64_t p = lane_xor64<(int)M>(v[q]);
      v[q] = ((p > v[q]) == keep_max) ? p : v[q];  // equal values: either is the result
    }
  }
}

// Every stage of runs of 2^KB, distances J, J / 2, ..., 1.
template <int EPT, int KB, uint32_t J, bool ALL_DESC = false>
__device__ __forceinline__ void sort_merge(uint64_t (&v)[EPT], uint32_t t, uint64_t (*c)[EPT * BLOCK], int& buf) {
  sort_stage<EPT, KB, J, ALL_DESC>(v, t, c, buf);
  if constexpr (J > 1u) sort_merge<EPT, KB, J / 2, ALL_DESC>(v, t, c, buf);
}

// Runs of 2^KB, 2^(KB+1), ..., 2^KTOP = EPT * WAVE entries, each wave's own entries: every
// exchange stays inside the wave (no barrier), and the last level leaves every wave's run
// in descending order.
template <int EPT, int KB, int KTOP>
__device__ __forceinline__ void sort_levels_wave(uint64_t (&v)[EPT], uint32_t t, uint64_t (*c)[EPT * BLOCK],
                                                 int& buf) {
  static_assert((1u << KTOP) == (uint32_t)EPT * WAVE, "one run per wave");
  if constexpr (KB < KTOP) {
    sort_merge<EPT, KB, (1u << KB) / 2>(v, t, c, buf);
    sort_levels_wave<EPT, KB + 1, KTOP>(v, t, c, buf);
  } else {
    sort_merge<EPT, KTOP, (1u << KTOP) / 2, true>(v, t, c, buf);
  }
}

// Merges the waves' descending runs of R = EPT * WAVE entries pairwise through LDS until one
// run of P = EPT * BLOCK entries remains; thread t ends with entries t*EPT .. t*EPT+EPT-1 of
// it. At each level a thread finds where its EPT outputs start by a binary search along
// the merge diagonal of its pair of runs (merge path), then takes them one by one; equal
// entries (only the zero padding) come from the first run first, both in the search and
// in the walk, so every output position is produced exactly once.
template <int EPT>
__device__ __forceinline__ void merge_wave_runs(uint64_t (&v)[EPT], uint32_t t, uint64_t (*c)[EPT * BLOCK]) {
  constexpr uint32_t P = (uint32_t)EPT * BLOCK, R = (uint32_t)EPT * WAVE;
  const uint32_t e0 = t * (uint32_t)EPT;
  int buf = 0;
#pragma unroll
  for (int q = 0; q < EPT; ++q) c[0][e0 + (uint32_t)q] = v[q];
  __syncthreads();
#pragma unroll
  for (uint32_t run = R; run < P; run *= 2u) {
    const uint64_t* A = c[buf] + (e0 & ~(2u * run - 1u));
    const uint64_t* B = A + run;
    const uint32_t d = e0 & (2u * run - 1u);  // outputs of the pair before this thread's
    uint32_t lo = d > run ? d - run : 0u, hi = d < run ? d : run;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;  // lo <= mid < hi: A[mid] and B[d - mid - 1] lie in their runs
      if (A[mid] >= B[d - mid - 1u]) lo = mid + 1u;
      else hi = mid;
    }
    uint32_t i = lo, j = d - lo;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      const uint64_t a = i < run ? A[i] : 0ull, b = j < run ? B[j] : 0ull;
      const bool take_a = j >= run || (i < run && a >= b);
      v[q] = take_a ? a : b;
      i += take_a ? 1u : 0u;
      j += take_a ? 0u : 1u;
    }
    if (2u * run < P) {
      uint64_t* dst = c[buf ^ 1];
#pragma unroll
      for (int q = 0; q < EPT; ++q) dst[e0 + (uint32_t)q] = v[q];
      __syncthreads();
      buf ^= 1;
    }
  }
}

// One row of the sorted output by the calling workgroup, through the LDS buffer c
// (2 EPT BLOCK 64-bit entries). Starts by reading the row's selected entries (written
// before the caller's last barrier), ends after its own writes.
template <int EPT>
__device__ __forceinline__ void sort_row(const float* __restrict__ scores, uint32_t row, uint32_t L, uint32_t N,
                                         uint32_t K, int32_t* __restrict__ out_idx, float* out_val,
                                         int32_t sentinel, uint64_t (*c)[EPT * BLOCK]) {
  const uint32_t t = threadIdx.x;
  const uint32_t n = L < K ? L : K;  // valid entries of the row
  int32_t* o = out_idx + (size_t)row * K;
  const uint32_t* x = reinterpret_cast<const uint32_t*>(scores) + (size_t)row * N;
  // For rows longer than K the selector left each selected key in out_val, beside its
  // index (read contiguously here); otherwise the scores are read at the indices (short
  // rows: the first L scores of the row, in order).
  const uint32_t* kin = (out_val != nullptr && L > K) ? reinterpret_cast<const uint32_t*>(out_val) + (size_t)row * K
                                                      : nullptr;
  float* val = out_val ? out_val + (size_t)row * K : nullptr;
  // Groups of four entries go through 16-byte loads and stores where the row's index,
  // key and value slots are 16-byte aligned and the group is entirely valid.
  const bool vec = (EPT % 4 == 0) && kin != nullptr &&
                   ((reinterpret_cast<uintptr_t>(o) | reinterpret_cast<uintptr_t>(kin)) & 15u) == 0u;
  uint64_t v[EPT];
#pragma unroll
  for (int g = 0; g < EPT; g += 4) {
    const uint32_t e0 = t * EPT + (uint32_t)g;
    if (EPT % 4 == 0 && vec && e0 + 3u < n) {
      const u32x4 iv = *reinterpret_cast<const u32x4*>(o + e0);
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kin + e0);
      v[g] = ((uint64_t)kv.x << 32) | (uint64_t)(0xFFFFFFFFu - iv.x);
      v[g + 1] = ((uint64_t)kv.y << 32) | (uint64_t)(0xFFFFFFFFu - iv.y);
      v[g + 2] = ((uint64_t)kv.z << 32) | (uint64_t)(0xFFFFFFFFu - iv.z);
      v[g + 3] = ((uint64_t)kv.w << 32) | (uint64_t)(0xFFFFFFFFu - iv.w);
      continue;
    }
#pragma unroll
    for (int q = g; q < g + 4 && q < EPT; ++q) {
      const uint32_t e = t * EPT + (uint32_t)q;
      v[q] = 0;
      if (e < n) {
        // The selector wrote an index in [0, L) here; the clamp only keeps reads in bounds.
        const uint32_t i = (uint32_t)o[e] < L ? (uint32_t)o[e] : 0u;
        const uint32_t k = kin != nullptr ? kin[e] : key_of_bits(x[i]);
        v[q] = ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - i);
      }
    }
  }
  __syncthreads();  // every key of the row is read before any thread overwrites out_val
  int buf = 0;
  constexpr int KTOP = EPT == 1 ? 6 : (EPT == 2 ? 7 : (EPT == 4 ? 8 : 9));
  sort_levels_wave<EPT, 1, KTOP>(v, t, c, buf);
  merge_wave_runs<EPT>(v, t, c);
  const bool vec_out = vec && val != nullptr && (reinterpret_cast<uintptr_t>(val) & 15u) == 0u;
  auto value_of = [](uint32_t key) { return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key); };
#pragma unroll
  for (int g = 0; g < EPT; g += 4) {
    const uint32_t e0 = t * EPT + (uint32_t)g;
    if (EPT % 4 == 0 && vec_out && e0 + 3u < n) {
      u32x4 iv, fv;
      iv.x = 0xFFFFFFFFu - (uint32_t)v[g];
      iv.y = 0xFFFFFFFFu - (uint32_t)v[g + 1];
      iv.z = 0xFFFFFFFFu - (uint32_t)v[g + 2];
      iv.w = 0xFFFFFFFFu - (uint32_t)v[g + 3];
      fv.x = __float_as_uint(value_of((uint32_t)(v[g] >> 32)));
      fv.y = __float_as_uint(value_of((uint32_t)(v[g + 1] >> 32)));
      fv.z = __float_as_uint(value_of((uint32_t)(v[g + 2] >> 32)));
      fv.w = __float_as_uint(value_of((uint32_t)(v[g + 3] >> 32)));
      *reinterpret_cast<u32x4*>(o + e0) = iv;
      *reinterpret_cast<u32x4*>(val + e0) = fv;
      continue;
    }
#pragma unroll
    for (int q = g; q < g + 4 && q < EPT; ++q) {
      const uint32_t e = t * EPT + (uint32_t)q;
      if (e < n) {
        o[e] = (int32_t)(0xFFFFFFFFu - (uint32_t)v[q]);
        if (val) val[e] = value_of((uint32_t)(v[q] >> 32));
      } else if (e < K) {
        o[e] = sentinel;
        if (val) val[e] = -__builtin_inff();
      }
    }
  }
}

template <int EPT>
__global__ __launch_bounds__(BLOCK) void sort_rows_kernel(const float* __restrict__ scores,
                                                          const int32_t* __restrict__ row_len,
                                                          uint32_t N, uint32_t K,
                                                          int32_t* __restrict__ out_idx,
                                                          float* out_val, int32_t sentinel) {
  __shared__ uint64_t c[2][(uint32_t)EPT * BLOCK];
  const uint32_t row = blockIdx.x;
  const int32_t len = row_len[row];
  uint32_t L = len < 0 ? 0u : (uint32_t)len;
  if (L > N) L = N;
  sort_row<EPT>(scores, row, L, N, K, out_idx, out_val, sentinel, c);
}

// One row, start to commit. Everything on the row's path is inlined: an out-of-line
// call per row would save and restore its callee-saved registers through scratch
// memory for every row.
template <bool STREAM_SAMPLE = false>
__device__ __forceinline__ void process_row_body(const Params& p, uint32_t row) {
  const uint32_t t = threadIdx.x;
  const int32_t len = p.row_len[row];
  uint32_t L = len < 0 ? 0u : (uint32_t)len;
  if (L > p.N) L = p.N;
  grow_t x = (grow_t)(p.scores) + (size_t)row * p.N;
  const RowOut out = row_out(p, row);
  if (t == 0) stat_add(p.ctl, TOPK_STAT_ROWS);
  phase_mark(p.phase, row, PH_START);
  if (L <= p.K) {
    for (uint32_t j = t; j < p.K; j += BLOCK) out.idx[j] = j < L ? (int32_t)j : p.sentinel;
    if (t == 0) stat_add(p.ctl, TOPK_STAT_SENTINEL);
    phase_mark(p.phase, row, PH_END);
    phase_path(p.phase, row, PATH_SENTINEL);
    return;
  }
  reset_row_state();
  const bool direct = (p.mode == TOPK_PATH_DIRECT) || (p.mode == TOPK_PATH_AUTO && L <= p.direct_max);
  if (direct) {
    if (t == 0) stat_add(p.ctl, TOPK_STAT_DIRECT);
    if (L <= (uint32_t)KEYS_CAP) direct_exact(x, L, p.K, out, p.ctl);
    else exact_full_row(x, L, p.K, 0u, KEY_MAX, out, p.ctl);
    phase_mark(p.phase, row, PH_END);
    phase_path(p.phase, row, PATH_DIRECT);
  } else if (p.mode == TOPK_PATH_RECOVERY) {
    if (t == 0) stat_add(p.ctl, TOPK_STAT_FORCED_RECOVERY);
    recover_row(p, row, x, L, 0u, KEY_MAX, out);
    phase_mark(p.phase, row, PH_END);
    phase_path(p.phase, row, PATH_FORCED_RECOVERY);
  } else {
    sampled_row<STREAM_SAMPLE>(p, row, x, L, out);
  }
}

// The sorted output's order, by the row's own workgroup once its selection is written
// (calls in which no row is handed to the recovery kernels): the candidate buffer,
// free by then, holds the sort's exchange buffer.
// Out of line (one copy for every kernel that holds it), taking scalars only.
__device__ __noinline__ void sort_row_here(const float* scores, uint32_t row, uint32_t L, uint32_t N, uint32_t K,
                                           int32_t* out, float* oval, int32_t sentinel) {
  __syncthreads();  // every output slot of the row is written
  auto* c = reinterpret_cast<uint64_t*>(g_s.buf);
  if (K <= (uint32_t)BLOCK) {
    sort_row<1>(scores, row, L, N, K, out, oval, sentinel, reinterpret_cast<uint64_t(*)[BLOCK]>(c));
  } else if (K <= 2u * BLOCK) {
    sort_row<2>(scores, row, L, N, K, out, oval, sentinel, reinterpret_cast<uint64_t(*)[2 * BLOCK]>(c));
  } else if (K <= 4u * BLOCK) {
    sort_row<4>(scores, row, L, N, K, out, oval, sentinel, reinterpret_cast<uint64_t(*)[4 * BLOCK]>(c));
  } else {
    sort_row<8>(scores, row, L, N, K, out, oval, sentinel, reinterpret_cast<uint64_t(*)[8 * BLOCK]>(c));
  }
}
static_assert(2 * 8 * BLOCK * sizeof(uint64_t) <= sizeof(uint32_t) * 2 * CAP, "the sort's exchange buffer fits the candidate buffer");

template <bool STREAM_SAMPLE = false>
__device__ __forceinline__ void process_row(const Params& p, uint32_t row) {
  // Sorted output: a row completed here is sorted here; a row handed to the recovery
  // kernels is sorted by the recovery finish kernel once complete. (Thread 0 clears the
  // flag and is the only writer; every thread reads it after the barrier below.)
  if (p.sort_rows && threadIdx.x == 0) g_s.queued = 0u;
  process_row_body<STREAM_SAMPLE>(p, row);
  if (p.sort_rows) {
    __syncthreads();
    if (!g_s.queued) sort_row_here(p.scores, row, row_length(p, row), p.N, p.K, (int32_t*)p.out, p.oval, p.sentinel);
  }
}

// The selector kernel. Persistent execution: a grid of resident workgroups pulls
// rows from a device ticket until none is left. Otherwise one workgroup per row,
// and the hardware dispatcher balances the rows over the CUs.
template <bool PERSISTENT>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void topk_rows_kernel(Params p) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  if (!PERSISTENT) {
    // All rows of the call start together, so their line samples are read in one
    // streaming phase: non-temporal loads read it fastest (512 rows of 1M: 0.398 ->
    // 0.383 ms per call). With persistent execution the rows are staggered and plain
    // loads let the hot sampled lines come back from cache (8192 rows of 1M were 1%
    // slower with non-temporal sample loads).
    if (t == 0) {
      s.row = (int32_t)blockIdx.x;
      stat_add(p.ctl, TOPK_STAT_ROW_PER_WG);
    }
    process_row<true>(p, blockIdx.x);
    return;
  }
  for (;;) {
    if (t == 0) s.row = (int32_t)atomicAdd(&p.ctl->row_ticket, 1u);
    __syncthreads();
    const uint32_t row = (uint32_t)s.row;
    if (row >= p.M) break;
    if (t == 0) stat_add(p.ctl, TOPK_STAT_PERSISTENT);
    process_row(p, row);
    __syncthreads();
  }
  // The last workgroup to leave rewinds the row ticket for the next call. Every
  // workgroup increments done_ticket only after its final ticket draw has returned,
  // so no draw can follow the rewind (both are device-scope atomics).
  if (t == 0) {
    const uint32_t d = atomicAdd(&p.ctl->done_ticket, 1u);
    if (d == gridDim.x - 1) {
      atomicExch(&p.ctl->row_ticket, 0u);
      atomicExch(&p.ctl->done_ticket, 0u);
    }
  }
}

// ------------------------------------------------------ cooperative recovery
//
// Exact full-row recovery of the queued rows, spread over the whole GPU. Each row
// is cut into REC_SEG-element work items. The histogram kernel bins every item
// into the row's global histogram over [lo, hi] (clamped at both ends). The
// collect kernel then derives, in every work item, the bin holding rank K,
// commits the item's keys above that bin and appends the bin's keys to the row's
// candidate buffer. The finish kernel (one workgroup per row) selects the
// remaining keys exactly from that buffer and commits them. Kernel boundaries
// order the three steps, so no cross-workgroup fences are needed. All three exit
// at once when the queue is empty; the finish kernel's last workgroup rewinds it.

// 16-byte chunks per thread per work item of SEG elements.
template <uint32_t SEG>
constexpr int rec_chunks() { return (int)(SEG / 4 / BLOCK + 1); }

struct RecHistSmem {
  uint32_t hist[NB];
};
__shared__ RecHistSmem g_rh;  // the histogram kernel's LDS state


template <uint32_t SEG>
__global__ __launch_bounds__(BLOCK) void recovery_hist_kernel(Params p) {
  constexpr int REC_CHUNKS = rec_chunks<SEG>();
  const uint32_t t = threadIdx.x;
  const uint32_t nq = min(p.ctl->qcount, p.qmax);
  const uint32_t per_row = (p.N + SEG - 1) / SEG;
  const uint32_t items = nq * per_row;
  for (uint32_t item = blockIdx.x; item < items; item += gridDim.x) {
    const uint32_t q = item / per_row;
    const uint32_t begin = (item - q * per_row) * SEG;
    RecSlot* r = p.rec + q;
    const uint32_t L = r->L;
    if (begin >= L || r->row >= p.M || L > p.N) continue;  // (a slot of a call that failed)
    if (r->mode != REC_HIST) continue;                     // the row's own pass located its bin
    const uint32_t n = min(SEG, L - begin);
    const uint32_t lo = r->lo, hi = r->hi;
    const uint32_t sh = shift_for(hi - lo);
    // The whole item is loaded at once (one memory latency per item): offsets are in
    // floats from the 16-byte chunk holding x[0]; chunks past the item read its last
    // chunk and their elements are masked.
    grow_t x = (grow_t)(p.scores) + (size_t)r->row * p.N + begin;
    const uint32_t off = (uint32_t)((uintptr_t)x & 15u) >> 2;
    grow_t ab = x - off;
    const uint32_t glast = (off + n - 1u) & ~3u;
    u32x4 v[REC_CHUNKS];
#pragma unroll
    for (int u = 0; u < REC_CHUNKS; ++u) {
      const uint32_t g = 4u * (t + (uint32_t)u * BLOCK);
      v[u] = load4(ab + (g < glast ? g : glast));
    }
    for (uint32_t i = t; i < (uint32_t)NB; i += BLOCK) g_rh.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < REC_CHUNKS; ++u) {
      const uint32_t g = 4u * (t + (uint32_t)u * BLOCK);
      const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t o = g + i;
        if (o >= off && o < off + n) {
          const uint32_t k = key_of_bits(w4[i]);
          const uint32_t d = k < lo ? 0u : (k - lo) >> sh;
          atomicAdd(&g_rh.hist[d < (uint32_t)(NB - 1) ? d : (uint32_t)(NB - 1)], 1u);
        }
      }
    }
    __syncthreads();
    for (uint32_t i = t; i < (uint32_t)NB; i += BLOCK) {
      const uint32_t c = g_rh.hist[i];
      if (c != 0) atomicAdd(&r->hist[i], c);
    }
    __syncthreads();
  }
}

// Per-item state of the collect kernel (its LDS is small, so many workgroups fit).
struct RecCollectSmem {
  uint32_t hist[NB];
  uint32_t wtmp[NWAVES];
  uint32_t wtmp2[NWAVES];
  uint32_t sel_bin, sel_above;
  uint32_t base_gt, base_bin;
};

__shared__ RecCollectSmem g_rc;

template <uint32_t SEG>
__global__ __launch_bounds__(BLOCK) void recovery_collect_kernel(Params p) {
  constexpr int REC_CHUNKS = rec_chunks<SEG>();
  RecCollectSmem& s = g_rc;
  const uint32_t t = threadIdx.x;
  const uint32_t K = p.K;
  const uint32_t nq = min(p.ctl->qcount, p.qmax);
  const uint32_t per_row = (p.N + SEG - 1) / SEG;
  const uint32_t items = nq * per_row;
  for (uint32_t item = blockIdx.x; item < items; item += gridDim.x) {
    const uint32_t q = item / per_row;
    const uint32_t begin = (item - q * per_row) * SEG;
    RecSlot* r = p.rec + q;
    const uint32_t L = r->L;
    if (begin >= L || r->row >= p.M || L > p.N) continue;  // (a slot of a call that failed)
    const uint32_t n = min(SEG, L - begin);
    // The item stays in registers; its loads are issued first so that they overlap
    // the boundary-bin search below. Then this thread's keys above the bin and in
    // the bin are counted, the item's output and candidate slots are reserved with
    // one atomic each, and written. Offsets are in floats from the 16-byte chunk
    // holding x[0].
    grow_t x = (grow_t)(p.scores) + (size_t)r->row * p.N + begin;
    const uint32_t off = (uint32_t)((uintptr_t)x & 15u) >> 2;
    grow_t ab = x - off;
    const uint32_t glast = (off + n - 1u) & ~3u;
    u32x4 v[REC_CHUNKS];
#pragma unroll
    for (int u = 0; u < REC_CHUNKS; ++u) {
      const uint32_t g = 4u * (t + (uint32_t)u * BLOCK);
      v[u] = load4(ab + (g < glast ? g : glast));
    }
    // The window of keys to gather, [blo, bhi], and whether the keys above it are
    // committed here: given by the row's own pass (REC_WINDOW), or derived in every item
    // from the completed histogram (REC_HIST).
    const uint32_t w = t / WAVE;
    uint32_t blo, bhi;
    bool fits = true, commit = true;
    if (r->mode == REC_WINDOW) {
      blo = r->bin_lo;
      bhi = r->bin_hi;
      commit = r->commit != 0u;
    } else {
      // The boundary bin, from the completed histogram (every item derives the same).
      uint32_t h[NB / BLOCK];
      uint32_t sum = 0;
#pragma unroll
      for (int j = 0; j < NB / BLOCK; ++j) {
        h[j] = r->hist[t * (NB / BLOCK) + j];
        sum += h[j];
        s.hist[t * (NB / BLOCK) + j] = h[j];
      }
      uint32_t incl = wave_incl_scan(sum);
      if (lane_id() == WAVE - 1) s.wtmp[w] = incl;
      if (t == 0) {
        s.sel_bin = 0;
        s.sel_above = 0;
      }
      __syncthreads();
      uint32_t before = 0, total = 0;
#pragma unroll
      for (int i = 0; i < NWAVES; ++i) {
        const uint32_t v = s.wtmp[i];
        before += ((uint32_t)i < w) ? v : 0u;
        total += v;
      }
      incl += before;
      const uint32_t hi_cnt = total - incl;
      if (hi_cnt < K && K <= hi_cnt + sum) {
        uint32_t cum = hi_cnt;
#pragma unroll
        for (int j = NB / BLOCK - 1; j >= 0; --j) {
          if (cum + h[j] >= K) {
            s.sel_bin = t * (NB / BLOCK) + j;
            s.sel_above = cum;
            break;
          }
          cum += h[j];
        }
      }
      __syncthreads();
      const uint32_t b = s.sel_bin, above = s.sel_above;
      const uint32_t cb = s.hist[b];
      const uint32_t lo = r->lo, hi = r->hi;
      const uint32_t sh = shift_for(hi - lo);
      const uint32_t braw = lo + (b << sh);
      blo = (b == 0) ? 0u : braw;
      const uint32_t wdt = (1u << sh) - 1u;
      bhi = (b == (uint32_t)(NB - 1)) ? KEY_MAX : braw + ((KEY_MAX - braw) < wdt ? (KEY_MAX - braw) : wdt);
      fits = cb <= (uint32_t)CAP;
      if (begin == 0 && t == 0) {  // one item per row records the bin for the finish kernel
        r->bin_above = above;
        r->bin_count = cb;
        r->bin_lo = blo;
        r->bin_hi = bhi;
      }
    }
    const RowOut out = row_out(p, r->row);
    uint32_t na = 0, nb = 0;
#pragma unroll
    for (int u = 0; u < REC_CHUNKS; ++u) {
      const uint32_t g = 4u * (t + (uint32_t)u * BLOCK);
      const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t o = g + i;
        const uint32_t k = key_of_bits(w4[i]);
        const bool ok = o >= off && o < off + n;
        na += (ok && commit && k > bhi) ? 1u : 0u;
        nb += (ok && fits && k >= blo && k <= bhi) ? 1u : 0u;
      }
    }
    uint32_t ia = wave_incl_scan(na), ib = wave_incl_scan(nb);
    if (lane_id() == WAVE - 1) {
      s.wtmp[w] = ia;
      s.wtmp2[w] = ib;
    }
    __syncthreads();
    uint32_t pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
    for (int i = 0; i < NWAVES; ++i) {
      const uint32_t va = s.wtmp[i], vb = s.wtmp2[i];
      pa += ((uint32_t)i < w) ? va : 0u;
      pb += ((uint32_t)i < w) ? vb : 0u;
      ta += va;
      tb += vb;
    }
    pa += ia - na;  // exclusive prefix of this thread
    pb += ib - nb;
    if (t == 0) {
      s.base_gt = ta ? atomicAdd(&r->out_gt, ta) : 0u;
      s.base_bin = tb ? atomicAdd(&r->cnt, tb) : 0u;
    }
    __syncthreads();
    pa += s.base_gt;
    pb += s.base_bin;
#pragma unroll
    for (int u = 0; u < REC_CHUNKS; ++u) {
      const uint32_t g = 4u * (t + (uint32_t)u * BLOCK);
      const uint32_t w4[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t o = g + i;
        const uint32_t k = key_of_bits(w4[i]);
        const bool ok = o >= off && o < off + n;
        const uint32_t e = begin + o - off;  // element index in the row
        if (ok && commit && k > bhi) {
          if (pa < K) out.put(pa, e, k);
          ++pa;
        }
        if (ok && fits && k >= blo && k <= bhi) {
          if (pb < (uint32_t)CAP) {
            r->cand_idx[pb] = e;
            r->cand_key[pb] = k;
          }
          ++pb;
        }
      }
    }
    __syncthreads();
  }
}

// One workgroup per queued row: resolve the boundary bin exactly and commit the
// remaining K - above keys. The kernel boundary orders it after every collect item.
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void recovery_finish_kernel(Params p) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x;
  const uint32_t K = p.K;
  const uint32_t nq = min(p.ctl->qcount, p.qmax);
  for (uint32_t q = blockIdx.x; q < nq; q += gridDim.x) {
    RecSlot* r = p.rec + q;
    if (r->row >= p.M || r->L > p.N) continue;  // (a slot of a call that failed)
    const bool window = r->mode == REC_WINDOW;
    const uint32_t above = r->bin_above;
    const uint32_t cb = window ? r->cnt : r->bin_count;  // (window: every key gathered, even past CAP)
    const uint32_t blo = r->bin_lo, bhi = r->bin_hi;
    const uint32_t need = K - above;
    const uint32_t L = r->L;
    grow_t x = (grow_t)(p.scores) + (size_t)r->row * p.N;
    const RowOut out = row_out(p, r->row);
    if (t == 0) {
      s.out_gt = above;
      s.out_tie = 0;
    }
    uint32_t T, gt2;
    if (window && cb < need) {
      // The window [tau2, tau1) of an underfilled row held fewer keys than it still
      // needs: the exact full-row select over the row, by this workgroup (it rewrites
      // every output slot).
      if (t == 0) stat_add(p.ctl, TOPK_STAT_INPLACE_FULL);
      exact_full_row(x, L, K, r->lo, r->hi, out, p.ctl);
    } else if (cb <= (uint32_t)FL_CAP) {
      if (t < cb) {
        s.fl_idx[t] = r->cand_idx[t];
        s.fl_key[t] = r->cand_key[t];
      }
      __syncthreads();
      const uint32_t rk = rank_in_list(s.fl_key, cb);
      const bool sel = rk < need;
      const uint32_t pp = wave_reserve(sel, &s.out_gt);
      if (sel && pp < K) out.put(pp, s.fl_idx[t], s.fl_key[t]);
    } else if (cb <= (uint32_t)CAP) {
      for (uint32_t i = t; i < cb; i += BLOCK) {
        s.buf[i] = r->cand_idx[i];
        s.buf[CAP + i] = r->cand_key[i];
      }
      __syncthreads();
      select_rank([&](auto&& f) {
        for (uint32_t i = threadIdx.x; i < cb; i += BLOCK) f(g_s.buf[CAP + i]);
      }, need, blo, bhi, T, gt2);
      commit_list(&s.buf[CAP], s.buf, cb, T, above + gt2, K, out);
    } else {
      // The boundary bin is wider than the buffer: narrow it with passes over the row.
      if (t == 0) stat_add(p.ctl, TOPK_STAT_FRONTIER_WIDE);
      __syncthreads();
      select_rank([&](auto&& f) {
        for_each_element(x, L, [&](uint32_t u, uint32_t) { f(key_of_bits(u)); });
      }, need, blo, bhi, T, gt2);
      const uint32_t gt_total = above + gt2;
      const uint32_t ties = K - gt_total;
      for_each_element(x, L, [&](uint32_t u, uint32_t e) {
        const uint32_t k = key_of_bits(u);
        const bool g = k > T && k <= bhi;
        const uint32_t pp = wave_reserve(g, &s.out_gt);
        if (g && pp < K) out.put(pp, e, k);
        const bool q_ = k == T;
        const uint32_t qq = wave_reserve(q_, &s.out_tie);
        if (q_ && qq < ties && gt_total + qq < K) out.put(gt_total + qq, e, k);
      });
    }
    __syncthreads();
    phase_mark(p.phase, r->row, PH_RECOVERED);
    if (p.sort_rows) {
      // Sorted output: the selector sorted the rows it completed; this row is sorted here.
      sort_row_here(p.scores, r->row, L, p.N, K, (int32_t*)p.out, p.oval, p.sentinel);
      __syncthreads();  // the sort's exchange area is free before the next row uses the LDS
    }
  }
  // The last workgroup to leave rewinds the queue for the next call; every
  // workgroup has read qcount before it increments rec_done.
  if (t == 0) {
    const uint32_t d = atomicAdd(&p.ctl->rec_done, 1u);
    if (d == gridDim.x - 1) {
      atomicExch(&p.ctl->qcount, 0u);
      atomicExch(&p.ctl->rec_done, 0u);
    }
  }
}

// -------------------------------------------------------------- row-split
//
// Row-split execution (the pages' KV-split, [PD] question 2; [AX]): when rows are
// few and long, one row's work is divided among several workgroups whose counts,
// candidates and histograms are merged for a final unit that certifies and refines.
// Here it is four kernels ordered by kernel boundaries (no workgroup waits on
// another):
//   split_sample (P_s x M)  each workgroup reads a share of the row's sampled lines
//                           whole into the row's global sample area;
//   split_select (M)        tau0 / tau1 once per row from the full sample;
//   split_pass   (P_p x M)  hot lines and the fused pass over a share of the
//                           512-byte periods; candidates, histogram and counts are
//                           merged into the row's state (one atomic per workgroup,
//                           one per non-empty bin);
//   split_finish (M)        certify, then refine and commit or queue for recovery.
// split_select runs only when the passing grid exceeds one round of resident
// workgroups (otherwise every passing workgroup selects the taus itself), and
// split_sample not at all for rows of at most 2048 sample periods or a single row
// (every passing workgroup then reads the row's element sample itself and passes the
// whole row). Rows the split does not apply to (L <= K, direct-exact, forced recovery,
// rows past the line-sample limit) are processed whole by split_finish. split_finish
// also rewinds the row state for the next call.

constexpr uint32_t RS_MAX_ROWS = 1024;  // rows per call the row-split state holds

struct RowSplitState {
  uint32_t whole;       // 1: the split does not apply, split_finish takes the row whole
  uint32_t mn_inv;      // bitwise NOT of the min sample key (atomicMax)
  uint32_t mx;          // max sample key (atomicMax)
  uint32_t c1;          // C(tau1): all admitted keys, even past CAP
  uint32_t c0;          // C(tau0)
  uint32_t t1key, t0key, t2key;
  uint32_t pad[24];
  uint32_t hist[NB];
  uint32_t cand_idx[CAP];
  uint32_t cand_key[CAP];
  uint32_t skey[LINE_SAMPLE_MAX];
  uint32_t lmax[LINE_SAMPLE_MAX];
};


__device__ __forceinline__ bool split_applies(const Params& p, uint32_t L) {
  if (L <= p.K) return false;
  if (p.mode == TOPK_PATH_DIRECT || p.mode == TOPK_PATH_RECOVERY) return false;
  if (p.mode == TOPK_PATH_AUTO && L <= p.direct_max) return false;
  if (p.stride != STRIDE) return false;
  return (L + STRIDE - 1) / STRIDE <= LINE_SAMPLE_MAX;
}

struct SplitSampleSmem {
  uint32_t mn, mx;
};
__shared__ SplitSampleSmem g_ssm;

__global__ __launch_bounds__(BLOCK) void split_sample_kernel(Params p) {
  const uint32_t t = threadIdx.x, part = blockIdx.x, row = blockIdx.y;
  RowSplitState* rs = p.rs + row;
  const uint32_t L = row_length(p, row);
  if (!split_applies(p, L)) {
    if (part == 0 && t == 0) rs->whole = 1u;
    return;
  }
  if (t == 0) {
    g_ssm.mn = KEY_MAX;
    g_ssm.mx = 0;
  }
  __syncthreads();
  const uint32_t n_s = (L + STRIDE - 1) / STRIDE;
  const uint32_t j0 = (uint32_t)((uint64_t)part * n_s / p.ps);
  const uint32_t j1 = (uint32_t)((uint64_t)(part + 1) * n_s / p.ps);
  grow_t x = (grow_t)(p.scores) + (size_t)row * p.N;
  uint32_t mn = KEY_MAX, mx = 0;
  sample_lines_range(x, L, j0, j1, (GLB uint32_t*)rs->skey, (GLB uint32_t*)rs->lmax, mn, mx);
  mn = wave_min_u32(mn);
  mx = wave_max_u32(mx);
  if (lane_id() == 0) {
    atomicMin(&g_ssm.mn, mn);
    atomicMax(&g_ssm.mx, mx);
  }
  __syncthreads();
  if (t == 0) {
    atomicMax(&rs->mn_inv, ~g_ssm.mn);
    atomicMax(&rs->mx, g_ssm.mx);
    if (part == 0) {
      stat_add(p.ctl, TOPK_STAT_ROWS);
      stat_add(p.ctl, TOPK_STAT_SAMPLED);
      stat_add(p.ctl, TOPK_STAT_ROWSPLIT);
    }
  }
}

__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void split_select_kernel(Params p) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x, row = blockIdx.x;
  RowSplitState* rs = p.rs + row;
  if (rs->whole) return;
  const uint32_t L = row_length(p, row);
  const uint32_t n_s = (L + STRIDE - 1) / STRIDE;
  // All of the sample's loads are issued before any is stored (one latency).
  uint32_t v[LM_PER_THREAD];
#pragma unroll
  for (int m = 0; m < LM_PER_THREAD; ++m) {
    const uint32_t i = t + (uint32_t)m * BLOCK;
    v[m] = i < n_s ? rs->skey[i] : 0u;
  }
#pragma unroll
  for (int m = 0; m < LM_PER_THREAD; ++m) {
    const uint32_t i = t + (uint32_t)m * BLOCK;
    if (i < n_s) s.buf[i] = v[m];
  }
  __syncthreads();
  // Line-sampled: the admission rank is tau1's.
  const uint32_t r1 = sample_rank(p.T1, n_s, L);
  uint32_t t0key, t1key, takey, t2key;
  select_taus(n_s, sample_rank(p.T0, n_s, L), r1, r1, sample_rank(p.T2, n_s, L), ~rs->mn_inv, rs->mx, t0key, t1key,
              takey, t2key);
  if (t == 0) {
    rs->t1key = t1key;
    rs->t0key = t0key;
    rs->t2key = t2key;
  }
}


__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void split_pass_kernel(Params p) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x, part = blockIdx.x, row = blockIdx.y;
  RowSplitState* rs = p.rs + row;
  const uint32_t L = row_length(p, row);
  if (p.split_elem) {
    // No sample kernel ran: the rows the split does not apply to are marked here.
    if (!split_applies(p, L)) {
      if (part == 0 && t == 0) rs->whole = 1u;
      return;
    }
  } else if (rs->whole) {
    return;
  }
  const uint32_t n_s = (L + STRIDE - 1) / STRIDE;
  grow_t x = (grow_t)(p.scores) + (size_t)row * p.N;
  uint32_t t0key, t1key, smax;
  if (p.split_elem) {
    // Short rows (at most 2048 sample periods): every passing workgroup reads the row's
    // element sample itself (the parts of a row share it through the cache) and selects
    // the taus from it, so no sample kernel runs. The pass then reads whole rows, as the
    // one-workgroup pass does for element-sampled rows; part 0 records the sample's
    // extremes and the taus for the finish.
    if (t == 0) {
      s.mn = KEY_MAX;
      s.mx = 0;
    }
    __syncthreads();
    uint32_t mn = KEY_MAX, mx = 0;
#pragma unroll 4
    for (uint32_t j = t; j < n_s; j += BLOCK) {
      const uint32_t k = key_of_bits(x[(size_t)j * STRIDE]);
      s.buf[j] = k;
      mn = min(mn, k);
      mx = max(mx, k);
    }
    block_minmax(mn, mx);
    const uint32_t smin = s.mn;
    smax = s.mx;
    uint32_t takey, t2key;
    const uint32_t r1 = sample_rank(p.T1, n_s, L);
    select_taus(n_s, sample_rank(p.T0, n_s, L), r1, r1, sample_rank(p.T2, n_s, L), smin, smax, t0key, t1key, takey,
                t2key);
    if (part == 0 && t == 0) {
      rs->mn_inv = ~smin;
      rs->mx = smax;
      rs->t1key = t1key;
      rs->t0key = t0key;
      rs->t2key = t2key;
      stat_add(p.ctl, TOPK_STAT_ROWS);
      stat_add(p.ctl, TOPK_STAT_SAMPLED);
      stat_add(p.ctl, TOPK_STAT_ROWSPLIT);
    }
  } else if (p.pass_taus) {
    // The taus from the whole sample, in every part (no separate select launch); part 0
    // records them for the finish.
    uint32_t v[LM_PER_THREAD];
#pragma unroll
    for (int m = 0; m < LM_PER_THREAD; ++m) {
      const uint32_t i = t + (uint32_t)m * BLOCK;
      v[m] = i < n_s ? rs->skey[i] : 0u;
    }
#pragma unroll
    for (int m = 0; m < LM_PER_THREAD; ++m) {
      const uint32_t i = t + (uint32_t)m * BLOCK;
      if (i < n_s) s.buf[i] = v[m];
    }
    __syncthreads();
    uint32_t takey, t2key;
    const uint32_t r1 = sample_rank(p.T1, n_s, L);
    select_taus(n_s, sample_rank(p.T0, n_s, L), r1, r1, sample_rank(p.T2, n_s, L), ~rs->mn_inv, rs->mx, t0key,
                t1key, takey, t2key);
    if (part == 0 && t == 0) {
      rs->t1key = t1key;
      rs->t0key = t0key;
      rs->t2key = t2key;
    }
    smax = rs->mx;
  } else {
    t1key = rs->t1key;
    t0key = rs->t0key;
    smax = rs->mx;
  }
  if (t1key == 0u) {
    // Every key is admitted at the lowest threshold: count the row as overflowing
    // so that it is recovered exactly.
    if (part == 0 && t == 0) atomicAdd(&rs->c1, (uint32_t)CAP + 1u);
    return;
  }
  const PassCtx c = pass_ctx(t1key, smax);
  // This part covers the sample periods [q0, q1): row elements [e0, e1), where period
  // P starts at offset 128 P from the 128-byte line below x (the last part runs to the
  // row's end, which may reach one element line past its last sampled period).
  const uint32_t q0 = (uint32_t)((uint64_t)part * n_s / p.pp);
  const uint32_t q1 = (uint32_t)((uint64_t)(part + 1) * n_s / p.pp);
  const uint32_t off4 = (uint32_t)((uintptr_t)x & 127u) >> 2;
  const uint32_t e0 = q0 == 0u ? 0u : 128u * q0 - off4;
  const uint32_t e1 = part == p.pp - 1 ? L : (q1 == 0u ? 0u : 128u * q1 - off4);
  if (p.split_elem) {
    reset_row_state();
    if (e1 > e0) {
      if (t1key >= 0x80000000u) fused_pass<true, false>(x + e0, e1 - e0, q1 - q0, c, e0);
      else fused_pass<false, false>(x + e0, e1 - e0, q1 - q0, c, e0);
    }
  } else {
    // Bitmap of this part's hot sampled lines (bit P - q0), as in the one-workgroup pass.
#pragma unroll
    for (int m = 0; m < LM_PER_THREAD; ++m) {
      const uint32_t j = t + (uint32_t)m * BLOCK;
      const uint64_t hb = __ballot(q0 + j < q1 && rs->lmax[q0 + j] >= t1key);
      if (lane_id() == 0) {
        s.fl_idx[j >> 5] = (uint32_t)hb;
        s.fl_idx[(j >> 5) + 1] = (uint32_t)(hb >> 32);
      }
    }
    reset_row_state();
    if (e1 > e0) {
      if (t1key >= 0x80000000u) fused_pass<true, true>(x + e0, e1 - e0, q1 - q0, c, e0);
      else fused_pass<false, true>(x + e0, e1 - e0, q1 - q0, c, e0);
    }
  }
  __syncthreads();
  // Merge into the row: one atomic reserves this workgroup's candidate range. C(tau0) is
  // counted among the part's listed keys (short of the truth only past the buffer, where
  // the row overflows anyway).
  const uint32_t n = s.cnt;
  const uint32_t keep = n < (uint32_t)CAP ? n : (uint32_t)CAP;
  count_admitted(keep, t0key, t1key);
  if (t == 0) {
    s.bcast = n ? atomicAdd(&rs->c1, n) : 0u;
    if (s.cnt0) atomicAdd(&rs->c0, s.cnt0);
  }
  __syncthreads();
  const uint32_t base = s.bcast;
  for (uint32_t i = t; i < keep; i += BLOCK) {
    if (base + i < (uint32_t)CAP) {
      rs->cand_idx[base + i] = s.buf[i];
      rs->cand_key[base + i] = s.buf[CAP + i];
    }
  }
  for (uint32_t b = t; b < (uint32_t)NB; b += BLOCK) {
    const uint32_t h = s.hist[b];
    if (h) atomicAdd(&rs->hist[b], h);
  }
}

__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(4)))
void split_finish_kernel(Params p) {
  Smem& s = g_s;
  const uint32_t t = threadIdx.x, row = blockIdx.x;
  RowSplitState* rs = p.rs + row;
  if (t == 0) s.row = (int32_t)row;
  if (rs->whole) {
    process_row(p, row);
  } else {
    phase_mark(p.phase, row, PH_START);
    const uint32_t L = row_length(p, row);
    grow_t x = (grow_t)(p.scores) + (size_t)row * p.N;
    const RowOut out = row_out(p, row);
    const uint32_t c1 = rs->c1, c0 = rs->c0;
    const uint32_t t1key = rs->t1key, t2key = rs->t2key;
    const uint32_t smin = ~rs->mn_inv, smax = rs->mx;
    if (c1 > (uint32_t)CAP) {
      if (t == 0) stat_add(p.ctl, TOPK_STAT_RECOVER_OVER);
      if (L <= p.inplace_max) {
        // The merged pass histogram (every part's admitted keys) locates the boundary bin.
        uint32_t thr = 0u, n_ge = 0u;
        if (t1key != 0u) {
          reset_row_state();
          for (uint32_t b = t; b < (uint32_t)NB; b += BLOCK) s.hist[b] = rs->hist[b];
          __syncthreads();
          thr = overflow_threshold(p.K, t1key, shift_for(smax - t1key), n_ge);
        }
        recover_in_place(x, L, p.K, n_ge <= (uint32_t)CAP ? thr : 0u, smax, t1key, smax, out, p.ctl);
      } else if (t1key != 0u) {
        reset_row_state();
        for (uint32_t b = t; b < (uint32_t)NB; b += BLOCK) s.hist[b] = rs->hist[b];
        __syncthreads();
        queue_overflow(p, row, x, L, t1key, shift_for(smax - t1key), smax, out);
      } else {
        // The lowest key (only a NaN pattern maps to it) admitted everything and the parts
        // built no histogram: the exact full-row select, here.
        recover_in_place(x, L, p.K, 0u, smax, t1key, smax, out, p.ctl);
      }
    } else if (c1 < p.K) {
      if (t == 0) stat_add(p.ctl, TOPK_STAT_RECOVER_UNDER);
      if (L <= p.inplace_max) recover_in_place(x, L, p.K, t2key, smax, smin, t1key, out, p.ctl);
      else queue_underfill(p, row, x, L, c1, t1key, t2key, smin, (const GLB uint32_t*)rs->cand_idx,
                           (const GLB uint32_t*)rs->cand_key, out);
    } else {
      if (t == 0) stat_add(p.ctl, c0 >= p.K ? TOPK_STAT_TAU0 : TOPK_STAT_TAU1);
      // The merged histogram and candidates move to LDS with all loads issued first.
      constexpr int HPT = NB / BLOCK, CPT = CAP / BLOCK;
      uint32_t h[HPT], ci[CPT], ck[CPT];
#pragma unroll
      for (int m = 0; m < HPT; ++m) h[m] = rs->hist[t + (uint32_t)m * BLOCK];
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const uint32_t i = t + (uint32_t)m * BLOCK;
        ci[m] = i < c1 ? rs->cand_idx[i] : 0u;
        ck[m] = i < c1 ? rs->cand_key[i] : 0u;
      }
      reset_row_state();
#pragma unroll
      for (int m = 0; m < HPT; ++m) s.hist[t + (uint32_t)m * BLOCK] = h[m];
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        const uint32_t i = t + (uint32_t)m * BLOCK;
        if (i < c1) {
          s.buf[i] = ci[m];
          s.buf[CAP + i] = ck[m];
        }
      }
      __syncthreads();
      refine_commit(c1, p.K, pass_ctx(t1key, smax), out, p.ctl);
    }
    phase_mark(p.phase, row, PH_END);
    phase_put(p.phase, row, PH_COUNTS, (unsigned long long)c1 | ((unsigned long long)c0 << 32));
    const bool rec = c1 > (uint32_t)CAP || c1 < p.K;
    phase_path(p.phase, row, PATH_SPLIT_FLAG | (rec ? (L <= p.inplace_max ? PATH_RECOVER_INPLACE : PATH_RECOVER_QUEUED)
                                                    : (c0 >= p.K ? PATH_TAU0 : PATH_TAU1)));
  }
  // Rewind the row's state for the next call (every read of it is done).
  __syncthreads();
  for (uint32_t b = t; b < (uint32_t)NB; b += BLOCK) rs->hist[b] = 0;
  if (t == 0) {
    rs->whole = 0;
    rs->mn_inv = 0;
    rs->mx = 0;
    rs->c1 = 0;
    rs->c0 = 0;
  }
}

__global__ void zero_stats_kernel(Control* ctl) {
  const uint32_t t = threadIdx.x;
  if (t < (uint32_t)TOPK_STAT_COUNT) ctl->stats[t] = 0ull;
}

// Plain streaming read for the measured-ceiling report: workgroup b reads the
// contiguous chunk [b*PROBE_CHUNK, (b+1)*PROBE_CHUNK) of 16-byte elements (4 MiB, a
// 1M-float row) with non-temporal loads, as the full-row pass does, four loads per lane
// in flight, and folds the bits so the loads cannot be elided. Workgroups are
// dispatched in address order, so the chunks read at any time are neighbours, as the
// rows of a selector call are. (A grid of a few hundred workgroups each streaming one
// far-apart span measured 8% slower on a 32 GiB buffer: 6.48 against 7.02 TB/s.)
constexpr uint64_t PROBE_CHUNK = 1ull << 18;
__global__ __launch_bounds__(BLOCK) void stream_read_probe_kernel(const float* __restrict__ x, uint64_t n,
                                                                  float* __restrict__ sink) {
  const u32x4* p4 = reinterpret_cast<const u32x4*>(x);
  const uint64_t nv = n >> 2;
  const uint64_t beg = (uint64_t)blockIdx.x * PROBE_CHUNK;
  const uint64_t end = beg + PROBE_CHUNK < nv ? beg + PROBE_CHUNK : nv;
  uint32_t acc = 0;
  uint64_t q = beg + threadIdx.x;
  for (; q + 3 * BLOCK < end; q += 4 * BLOCK) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(&p4[q + (uint64_t)u * BLOCK]);
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; q < end; q += BLOCK) {
    const u32x4 a = __builtin_nontemporal_load(&p4[q]);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (blockIdx.x == gridDim.x - 1) {
    const uint32_t* xu = reinterpret_cast<const uint32_t*>(x);
    for (uint64_t i = 4 * nv + threadIdx.x; i < n; i += BLOCK) acc ^= xu[i];
  }
  acc = wave_max_u32(acc);  // any combine that depends on every lane keeps the loads live
  __shared__ uint32_t w[NWAVES];
  if (lane_id() == 0) w[threadIdx.x / WAVE] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t v = 0;
    for (int i = 0; i < NWAVES; ++i) v ^= w[i];
    sink[blockIdx.x & 4095u] = __uint_as_float(v);
  }
}

// ------------------------------------------------------------------- host side

struct DevState {
  bool ready = false;
  int n_cu = 0;
  int occ = 0;          // resident selector workgroups per CU
  int occ_rec = 0;      // resident recovery-collect workgroups per CU
  Control* ctl = nullptr;
  RecSlot* rec = nullptr;
  RowSplitState* rs = nullptr;  // row-split state for rs_rows rows
  uint32_t qmax = QMAX;         // recovery slots
  int64_t rs_rows = RS_MAX_ROWS;
};

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
DevState g_dev[MAX_DEVICES];
std::atomic<int> g_mode{TOPK_PATH_AUTO};
std::atomic<int> g_exec{TOPK_EXEC_AUTO};
// Proposal parameters: sample stride and the two candidate targets in thousandths of K.
std::atomic<int> g_stride{(int)STRIDE};
std::atomic<int> g_rho0{1500};
std::atomic<int> g_rho1{1750};
std::atomic<int> g_rhoa{2250};  // deeper admission target of element-sampled rows; 0: off
// Per-row phase recording (measurement hook): device buffer and its row capacity.
std::atomic<unsigned long long*> g_phase_buf{nullptr};
std::atomic<int64_t> g_phase_rows{0};
thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TOPK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Launch limits of a device: compute units and resident workgroups per CU of the
// selector and recovery kernels (queries only; nothing is allocated).
int launch_limits(int dev, DevState* st) {
  int n_cu = 0, occ = 0, occ_rec = 0;
  hipError_t e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(topk_rows_kernel<true>),
                                                   BLOCK, 0);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  if (occ < 1) return fail(TOPK_ERR_HIP, "selector kernel cannot be resident (occupancy %d)", occ);
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ_rec, reinterpret_cast<const void*>(recovery_finish_kernel),
                                                   BLOCK, 0);
  if (e != hipSuccess) return hip_fail(e, "hipOccupancyMaxActiveBlocksPerMultiprocessor");
  if (occ_rec < 1) return fail(TOPK_ERR_HIP, "recovery kernel cannot be resident");
  st->n_cu = n_cu;
  st->occ = occ;
  st->occ_rec = occ_rec;
  return TOPK_OK;
}

// Returns the current device's state, creating it when allowed.
int get_state(bool capturing, DevState** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(TOPK_ERR_HIP, "device index %d unsupported", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  DevState& st = g_dev[dev];
  if (!st.ready) {
    if (capturing)
      return fail(TOPK_ERR_WORKSPACE,
                  "workspace not created on device %d; call topk_exact_reserve before capturing", dev);
    DevState lim;
    int rc = launch_limits(dev, &lim);
    if (rc != TOPK_OK) return rc;
    // One allocation: the control block, the recovery slots, then the row-split state
    // (about 160 MB in all), so that no later call allocates.
    const size_t rec_off = (sizeof(Control) + 255) / 256 * 256;
    const size_t rs_off = (rec_off + sizeof(RecSlot) * QMAX + 255) / 256 * 256;
    const size_t bytes = rs_off + sizeof(RowSplitState) * RS_MAX_ROWS;
    char* ws = nullptr;
    e = hipMalloc(reinterpret_cast<void**>(&ws), bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    e = hipMemset(ws, 0, bytes);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      (void)hipFree(ws);
      return hip_fail(e, "workspace initialisation");
    }
    st.n_cu = lim.n_cu;
    st.occ = lim.occ;
    st.occ_rec = lim.occ_rec;
    st.ctl = reinterpret_cast<Control*>(ws);
    st.rec = reinterpret_cast<RecSlot*>(ws + rec_off);
    st.rs = reinterpret_cast<RowSplitState*>(ws + rs_off);
    st.ready = true;
  }
  *out = &st;
  return TOPK_OK;
}

// One-shot selector timing for the next call on this host thread.
thread_local hipEvent_t g_time_start = nullptr, g_time_stop = nullptr;

int stream_capturing(hipStream_t stream, bool* capturing) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(stream, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  *capturing = cs != hipStreamCaptureStatusNone;
  return TOPK_OK;
}

// Scratch of the allocation-free entry point (topk_exact_noalloc): a control block, NA_QMAX
// cooperative-recovery slots and row-split state for NA_RS_ROWS rows, laid out like the
// workspace. It exists once per GPU from load to process end, zero at load. In host code
// `scratch` names a host-side stand-in, never the device memory: the device address comes
// from hipGetSymbolAddress once per device (noalloc_state) and only that address is used.
constexpr uint32_t NA_QMAX = 64;
constexpr int64_t NA_RS_ROWS = 64;
constexpr size_t NA_REC_OFF = (sizeof(Control) + 255) / 256 * 256;
constexpr size_t NA_RS_OFF = (NA_REC_OFF + sizeof(RecSlot) * NA_QMAX + 255) / 256 * 256;
constexpr size_t NA_SCRATCH_BYTES = NA_RS_OFF + sizeof(RowSplitState) * NA_RS_ROWS;
static_assert(NA_SCRATCH_BYTES <= (16u << 20), "the allocation-free scratch stays under 16 MiB");

}  // namespace

static __device__ __align__(256) unsigned char scratch[NA_SCRATCH_BYTES];

namespace {

DevState g_noalloc[MAX_DEVICES];  // per device: limits and the device address of `scratch`

// The allocation-free state of the current device: launch limits (queries only) and the
// device address of `scratch`, looked up once per device with that device current.
int noalloc_state(DevState** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(TOPK_ERR_HIP, "device index %d unsupported", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  DevState& st = g_noalloc[dev];
  if (!st.ready) {
    DevState lim;
    int rc = launch_limits(dev, &lim);
    if (rc != TOPK_OK) return rc;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (ptr == nullptr) return fail(TOPK_ERR_HIP, "hipGetSymbolAddress(scratch) gave no address");
    char* base = static_cast<char*>(ptr);
    st.n_cu = lim.n_cu;
    st.occ = lim.occ;
    st.occ_rec = lim.occ_rec;
    st.ctl = reinterpret_cast<Control*>(base);
    st.rec = reinterpret_cast<RecSlot*>(base + NA_REC_OFF);
    st.rs = reinterpret_cast<RowSplitState*>(base + NA_RS_OFF);
    st.qmax = NA_QMAX;
    st.rs_rows = NA_RS_ROWS;
    st.ready = true;
  }
  *out = &st;
  return TOPK_OK;
}

}  // namespace

// The indexer score producer's host-side checks and launch (indexer_scores.hip).
int topk_indexer_check(const uint8_t* q, const uint8_t* k, const float* w, const int32_t* row_len,
                       int64_t T, int64_t S, int32_t H, int32_t D, const float* out);
int topk_indexer_launch(const uint8_t* q, const uint8_t* k, const float* w, const int32_t* row_len,
                        int64_t T, int64_t S, int32_t H, float* out, hipStream_t stream);

// Records an error text for topk_exact_last_error() on behalf of the library's other
// translation units (the indexer score producer).
__attribute__((visibility("hidden"))) int topk_record_error(int code, const char* text) {
  return fail(code, "%s", text);
}

namespace {

// Argument checks of a selector call (no device state is touched).
int selector_args(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc, int32_t K,
                  const int32_t* out_idx, int32_t sentinel) {
  if (M < 0) return fail(TOPK_ERR_BAD_SHAPE, "M = %lld is negative", (long long)M);
  if (N_alloc < 1 || N_alloc > INT32_MAX)
    return fail(TOPK_ERR_BAD_SHAPE, "N_alloc = %lld outside [1, INT32_MAX]", (long long)N_alloc);
  if (K < 1 || K > TOPK_K_MAX) return fail(TOPK_ERR_BAD_K, "K = %d outside [1, %d]", K, TOPK_K_MAX);
  if (M > INT32_MAX) return fail(TOPK_ERR_BAD_SHAPE, "M = %lld exceeds INT32_MAX", (long long)M);
  if (M > 0 && (N_alloc > INT64_MAX / M || (int64_t)K > INT64_MAX / M))
    return fail(TOPK_ERR_BAD_SHAPE, "M*N_alloc or M*K overflows");
  if (sentinel >= 0 && (int64_t)sentinel < N_alloc)
    return fail(TOPK_ERR_BAD_SENTINEL, "sentinel %d lies inside [0, N_alloc = %lld)", sentinel,
                (long long)N_alloc);
  if (M == 0) return TOPK_OK;
  if (!scores || !row_len || !out_idx) return fail(TOPK_ERR_NULL_POINTER, "null scores/row_len/out_idx");
  if ((reinterpret_cast<uintptr_t>(scores) & 3u) != 0)
    return fail(TOPK_ERR_BAD_ARG, "scores is not 4-byte aligned");
  return TOPK_OK;
}

// Host-side checks of a selector call and the device state it runs with. Returns an error
// before anything is enqueued; on success *st_out is null when there is nothing to
// launch (M == 0).
int selector_check(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc, int32_t K,
                   int32_t* out_idx, int32_t sentinel, hipStream_t stream, bool* capturing_out,
                   DevState** st_out) {
  *st_out = nullptr;
  *capturing_out = false;
  int rc = selector_args(scores, row_len, M, N_alloc, K, out_idx, sentinel);
  if (rc != TOPK_OK || M == 0) return rc;  // *st_out stays null for M == 0: nothing to launch
  bool capturing = false;
  rc = stream_capturing(stream, &capturing);
  if (rc != TOPK_OK) return rc;
  DevState* st = nullptr;
  rc = get_state(capturing, &st);
  if (rc != TOPK_OK) return rc;
  *capturing_out = capturing;
  *st_out = st;
  return TOPK_OK;
}


// Enqueues the selector and recovery kernels of a checked call on the state st (the
// workspace, or the allocation-free entry point's scratch). `timing`: the call may take
// the armed timing events (not under capture).
// `okey`: device [M][K], receives each selected element's key in its output slot
// (sorted output), or null. `sort_here` (sorted output): set to whether the selector
// kernels also sort every row (then no separate sort follows), or null.
int selector_launch(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc, int32_t K,
                    int32_t* out_idx, int32_t sentinel, hipStream_t stream, bool timing, DevState* st,
                    uint32_t* okey = nullptr, bool* sort_here = nullptr) {
  int rc = TOPK_OK;
  Params p;
  p.scores = scores;
  p.row_len = row_len;
  p.out = out_idx;
  p.ctl = st->ctl;
  p.M = (uint32_t)M;
  p.N = (uint32_t)N_alloc;
  p.K = (uint32_t)K;
  p.sentinel = sentinel;
  // Targets ceil(rho * K) with rho in thousandths: 1.5 K and 1.75 K by default (3072 and
  // 3584 at K = 2048). Away from that operating point they are bounded: at least 12 and
  // 16 samples' worth (a sample rank below that estimates its quantile too coarsely:
  // 5% of 128K rows underfilled at K = 512 with tau1 at rank 7), and at most 5/8 and 3/4
  // of the candidate buffer (the spread of C(tau1) is about 1/sqrt(rank) of it: at
  // K = 4096, 1.75 K = 7168 overflowed 8192 slots in 17% of 1M rows).
  {
    const int64_t s_ = g_stride.load();
    int64_t t0 = ((int64_t)g_rho0.load() * K + 999) / 1000, t1 = ((int64_t)g_rho1.load() * K + 999) / 1000;
    t0 = t0 < 12 * s_ ? 12 * s_ : t0;
    t1 = t1 < 16 * s_ ? 16 * s_ : t1;
    t0 = t0 > 5 * CAP / 8 ? 5 * CAP / 8 : t0;
    t1 = t1 > 3 * CAP / 4 ? 3 * CAP / 4 : t1;
    p.T0 = (uint32_t)t0;
    p.T1 = (uint32_t)(t1 > t0 ? t1 : t0);
  }
  // Recovery threshold of an underfilled row: a deeper sample rank, about 2.9 K admitted
  // keys at K = 2048 (halfway from T1 to the buffer, at most max(3 K, 2 T1)). After an
  // underfill at tau1 the row holds about C(tau1) + (r2 - r1) L / n_s keys above it.
  {
    const uint32_t half = (p.T1 + (uint32_t)CAP) / 2u;
    const uint32_t lim = 3u * (uint32_t)K > 2u * p.T1 ? 3u * (uint32_t)K : 2u * p.T1;
    const uint32_t t2 = half < lim ? half : lim;
    p.T2 = t2 > p.T1 ? t2 : p.T1;
  }
  // Admission target of rows sampled one element per period: 2.25 K by default (4608 at
  // K = 2048), used where it lies strictly between T1 and T2 and within 9/16 of the
  // candidate buffer, else T1. For a row of exchangeable scores the chance that its
  // admitted count falls short of K or exceeds the buffer (hypergeometric tails; 1024
  // samples of 128K) is 3.7e-3 at T1 (rank 28) and 4e-5 at 4608 (rank 36) at K = 2048;
  // at K >= 3000 no deeper rank lowers it, and 2.25 K passes the buffer bound there.
  {
    const int64_t ra = g_rhoa.load();
    const int64_t ta = (ra * K + 999) / 1000;
    p.TA = (ta > (int64_t)p.T1 && ta < (int64_t)p.T2 && ta <= 9 * CAP / 16) ? (uint32_t)ta : p.T1;
  }
  // Rows that need exact recovery and are short are recovered by their own workgroup
  // with one more pass (at most 256 KB; 1 MB in row-split calls, which have few rows);
  // longer ones by the cooperative recovery kernels, which then run after the selector.
  // Measured on MI355X (graph replays): 8192 x 64K bf16 rows 0.587 -> 0.558 ms per call
  // and 64 split rows of 128K 49 -> 45 us in place, while 512 x 128K rows in lockstep lose
  // 3-5 us (the recovering workgroup streams its row alone at the end of the call). Forced
  // recovery always takes the cooperative kernels.
  p.stride = (uint32_t)g_stride.load();
  p.direct_max = DIRECT_MAX_DEFAULT;
  p.mode = g_mode.load();
  p.rec = st->rec;
  p.qmax = st->qmax;
  p.rs = nullptr;
  p.phase = (timing && M <= g_phase_rows.load()) ? g_phase_buf.load() : nullptr;
  p.okey = okey;
  p.sort_rows = 0;
  p.oval = nullptr;
  p.ps = 1;
  p.pp = 1;
  p.pass_taus = 0;
  p.split_elem = 0;
  // Execution by shape. Row-split when rows are few and long: their scan and
  // sampling are divided among several workgroups. Measured on MI355X (512 resident
  // slots, graph replays): for rows of 1M, row-split takes 44-62 us for 1-32 rows
  // against 224-241 us, 146 against 240 us at 128 rows, about even at 256 and slower
  // at 512, where one workgroup per row already fills the chip and the extra kernel
  // boundaries and merges cost more than they save; for rows of 128K it wins up to
  // 64 rows (44 against 52 us) and loses from 128 (60 against 55 us). So: at most a
  // quarter of the resident slots for rows of 256K and more, an eighth for rows of
  // 64K-256K. Persistent execution
  // for many long rows per resident workgroup. One workgroup per row otherwise
  // (equal to persistent on 0.5-1M-wide rows, faster on short rows, where the
  // per-row loop overhead is not amortised).
  const int64_t resident = (int64_t)st->occ * st->n_cu;
  const int ex = g_exec.load();
  // The deeper admission pays where a row's exact recovery would lengthen the call: at
  // most one row per resident workgroup (512 x 128K: 95.5 -> 79.9 us per call with it and
  // in-place recovery). With more rows per workgroup a rare recovery is absorbed by the
  // workgroup's other rows, and the extra candidates cost more than it saves: 4096 rows
  // of 32K and 64K bf16 take 0.197 and 0.265 ms admitting at tau1, 0.203 and 0.271 ms
  // admitting down to tau_a.
  if (M > resident) p.TA = p.T1;
  // Line sampling reads the sampled lines whole and skips them in the full pass; a
  // sampled line is read again when its maximum reaches tau1 ("hot"). With about T1
  // admitted elements in a row of L, a 32-element line is hot with probability of
  // roughly 32 T1 / L, and the saving (a quarter of the row) shrinks with that
  // re-read share. Auto dispatch uses it where at most about one sampled line in four
  // is expected hot: L >= 128 T1, i.e. n_s >= T1 sample lines (measured: 4096 x 512K
  // 1.507 -> 1.485 ms; 512 x 128K and 64K rows, where most lines are hot, lose with
  // it). A forced sampled path keeps it wherever it applies.
  p.line_min = (p.mode == TOPK_PATH_SAMPLED) ? 0u : p.T1;
  const bool split = M <= st->rs_rows &&
               (ex == TOPK_EXEC_ROWSPLIT || p.mode == TOPK_PATH_ROWSPLIT ||
                (ex == TOPK_EXEC_AUTO && N_alloc >= ROWSPLIT_MIN_N &&
                 (N_alloc >= 4 * ROWSPLIT_MIN_N ? 4 * M <= resident : 8 * M <= resident)));
  p.inplace_max = g_mode.load() == TOPK_PATH_RECOVERY ? 0u : (split ? INPLACE_MAX_SPLIT : INPLACE_MAX);
  // With the deeper admission, rows sampled one element per period (at stride 128 those
  // with fewer than line_min sample periods) need exact recovery about once in 25000 rows
  // of 128K, so they are recovered in place at any length: a call whose rows are all such
  // rows launches no recovery kernels (512 x 128K: 86 -> 80 us per call), and the rare row
  // that does recover streams its row once more on its own. The same holds where tau1
  // itself targets at least 2 K (K <= 1024, whose targets are floored at 16 sample
  // ranks): 512 x 128K at K = 512 82.0 -> 75.2 us.
  if (!split && p.inplace_max != 0u && (p.TA > p.T1 || p.T1 >= 2u * (uint32_t)K) && p.stride == STRIDE &&
      p.line_min > 1u) {
    const uint32_t elem_max = (p.line_min - 1u) * STRIDE;
    if (elem_max > p.inplace_max) p.inplace_max = elem_max;
  }
  const bool persistent = !split && (ex == TOPK_EXEC_PERSISTENT ||
                                      (ex == TOPK_EXEC_AUTO && M >= 4 * resident && N_alloc >= 262144));
  // Sorted output: each workgroup sorts a row once it completes it, overlapping the other
  // rows' passes (the selector's workgroup for the rows it completes, the recovery finish
  // kernel's for the rows handed to it), in calls of at most one row per resident
  // workgroup where no row can be handed over, and in persistent calls; otherwise a sort
  // kernel follows. Measured on MI355X (graph replays, sorted call): 512 x 128K 94.8 ->
  // 90.5 us and 256 x 8K 26.5 -> 24.7 us sorted here; persistent 8192 x 1M 5.46 -> 5.43 ms
  // and 4096 x 512K 1.495 -> 1.480 ms. Not kept: 512 x 1M with its queued rows sorted by
  // the recovery finish kernel (388 -> 391 us), and 8192 x 64K rows, sixteen per
  // workgroup, one workgroup per row (622.7 -> 657.4 us).
  if (sort_here != nullptr) {
    *sort_here = !split && (persistent || ((int64_t)p.inplace_max >= N_alloc && M <= resident));
    if (*sort_here) {
      p.sort_rows = 1;
      p.oval = reinterpret_cast<float*>(okey);
    }
  }
  hipError_t e;
  hipEvent_t ev_start = nullptr, ev_stop = nullptr;
  if (timing && g_time_start) {
    ev_start = g_time_start;
    ev_stop = g_time_stop;
    g_time_start = g_time_stop = nullptr;
    // Both events are checked before anything is enqueued: once the selector kernel is,
    // the recovery kernels must follow it (they rewind the queue it fills).
    e = hipEventQuery(ev_stop);
    if (e != hipSuccess && e != hipErrorNotReady) return hip_fail(e, "timing stop event");
    e = hipEventRecord(ev_start, stream);
    if (e != hipSuccess) return hip_fail(e, "hipEventRecord(start)");
  }
  if (split) {
    // Workgroups per row: enough units to keep every resident slot busy several times
    // over, at most `cap` per row, and no unit smaller than `unit_p` periods (pass) /
    // `unit_s` sampled lines (sample). Measured on MI355X (graph replays, median call):
    // a cap of 64 rows for 1-4 rows of 1M takes 1 row from 50.3 to 42.0 us and 4 rows from
    // 52.1 to 43.3 us (16 and 64 rows unchanged at 16); units of 64 periods / lines for at
    // most 16 rows of up to 256K take 1 row of 128K from 37.4 to 33.5 us and 16 rows from
    // 38.2 to 34.9 us, while 64 rows lose with them (43.8 -> 54.0 us).
    const int64_t n_s_max = (N_alloc + STRIDE - 1) / STRIDE;
    const int64_t cap = M <= 4 ? 64 : (M <= 8 ? 32 : 16);
    const bool small_units = M <= 16 && n_s_max <= 2048;
    const int64_t unit_p = small_units ? 64 : 170, unit_s = small_units ? 64 : 256;
    int64_t pp = (4 * resident + M - 1) / M, ps = (2 * resident + M - 1) / M;
    pp = pp < 1 ? 1 : (pp > cap ? cap : pp);
    ps = ps < 1 ? 1 : (ps > cap ? cap : ps);
    const int64_t pp_cap = n_s_max / unit_p > 1 ? n_s_max / unit_p : 1;
    const int64_t ps_cap = n_s_max / unit_s > 1 ? n_s_max / unit_s : 1;
    p.pp = (uint32_t)(pp < pp_cap ? pp : pp_cap);
    p.ps = (uint32_t)(ps < ps_cap ? ps : ps_cap);
    p.rs = st->rs;
    // When the passing grid fits in one round of resident workgroups, each of them
    // selects its row's taus from the sample (a few microseconds, overlapped across the
    // grid) instead of waiting for a select kernel. Measured on MI355X (selector kernels,
    // graph replays): 1-16 rows of 128K and 1-4 rows of 1M gain 1.1-1.6 us, 64 rows of
    // 128K and 16 rows of 1M 0.6-0.9 us. A larger grid repeats that work in later rounds,
    // and 64 rows of 1M lose 6 us with it.
    p.pass_taus = (int64_t)p.pp * M <= resident ? 1u : 0u;
    // With the taus selected in the passing workgroups, each of them can read the row's
    // element sample itself, so that no sample kernel is launched; the pass then reads the
    // whole row (no line skipping). Measured on MI355X (graph replays, median call): rows
    // of 128K, 1 / 4 / 16 / 64 of them, 30.4 / 31.0 / 31.8 / 39.1 -> 25.1 / 25.6 / 26.8 /
    // 37.4 us (most of their sampled lines are hot anyway); one 1M row 37.9 -> 35.0 us,
    // but 4 and 16 rows of 1M lose 2 and 9 us (every part re-reads 8192 samples, and the
    // skipped cold lines are read). So: rows of at most 2048 sample periods, or one row.
    p.split_elem = (p.pass_taus && (n_s_max <= 2048 || M == 1)) ? 1u : 0u;
    if (!p.split_elem) hipLaunchKernelGGL(split_sample_kernel, dim3(p.ps, (unsigned)M), dim3(BLOCK), 0, stream, p);
    if (!p.pass_taus) hipLaunchKernelGGL(split_select_kernel, dim3((unsigned)M), dim3(BLOCK), 0, stream, p);
    hipLaunchKernelGGL(split_pass_kernel, dim3(p.pp, (unsigned)M), dim3(BLOCK), 0, stream, p);
    hipLaunchKernelGGL(split_finish_kernel, dim3((unsigned)M), dim3(BLOCK), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch row-split kernels");
  } else {
    if (persistent) {
      const unsigned grid = (unsigned)(M < resident ? M : resident);
      hipLaunchKernelGGL(topk_rows_kernel<true>, dim3(grid), dim3(BLOCK), 0, stream, p);
    } else {
      hipLaunchKernelGGL(topk_rows_kernel<false>, dim3((unsigned)M), dim3(BLOCK), 0, stream, p);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch topk_rows_kernel");
  }
  // From here on every step is enqueued even if one fails; the first error is returned.
  if (ev_stop) {
    e = hipEventRecord(ev_stop, stream);
    if (e != hipSuccess) rc = hip_fail(e, "hipEventRecord(stop)");
  }
  // Exact recovery of the rows the selector queued (they exit at once if none). Only rows
  // longer than p.inplace_max are queued: with no such row the recovery kernels are not
  // launched at all. At most min(M, qmax) rows can be queued, so small calls launch
  // correspondingly small grids.
  if ((int64_t)p.inplace_max >= N_alloc) return rc;
  const int64_t rec_rows = M < (int64_t)st->qmax ? M : (int64_t)st->qmax;
  // Work items of 4K elements for rows of up to 256K (more workgroups on the few items of
  // a short row: 512 x 128K 99 -> 94 us per call), of 16K for longer rows (fewer items each
  // workgroup walks in turn: 4K items cost 8192 x 1M rows about 20 us more).
  const bool short_items = N_alloc <= REC_SHORT_MAX_N;
  const int64_t seg = short_items ? REC_SEG_SHORT : REC_SEG;
  const int64_t rec_items = rec_rows * ((N_alloc + seg - 1) / seg);
  const unsigned rec_grid = (unsigned)(rec_items < (int64_t)st->n_cu * 4 ? rec_items : (int64_t)st->n_cu * 4);
  // Only forced recovery queues rows with nothing known about their K-th key; every
  // other queued row comes with the window its own pass located, and needs no histogram.
  if (p.mode == TOPK_PATH_RECOVERY) {
    if (short_items) hipLaunchKernelGGL(recovery_hist_kernel<REC_SEG_SHORT>, dim3(rec_grid), dim3(BLOCK), 0, stream, p);
    else hipLaunchKernelGGL(recovery_hist_kernel<REC_SEG>, dim3(rec_grid), dim3(BLOCK), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess && rc == TOPK_OK) rc = hip_fail(e, "launch recovery_hist_kernel");
  }
  if (short_items) hipLaunchKernelGGL(recovery_collect_kernel<REC_SEG_SHORT>, dim3(rec_grid), dim3(BLOCK), 0, stream, p);
  else hipLaunchKernelGGL(recovery_collect_kernel<REC_SEG>, dim3(rec_grid), dim3(BLOCK), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess && rc == TOPK_OK) rc = hip_fail(e, "launch recovery_collect_kernel");
  const int64_t fin_cap = (int64_t)st->n_cu * st->occ_rec;
  const unsigned fin_grid = (unsigned)(rec_rows < fin_cap ? rec_rows : fin_cap);
  hipLaunchKernelGGL(recovery_finish_kernel, dim3(fin_grid), dim3(BLOCK), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess && rc == TOPK_OK) rc = hip_fail(e, "launch recovery_finish_kernel");
  return rc;
}


}  // namespace

extern "C" {

int topk_exact(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc, int32_t K,
               int32_t* out_idx, int32_t sentinel, hipStream_t stream) {
  g_err[0] = '\0';
  bool capturing = false;
  DevState* st = nullptr;
  const int rc = selector_check(scores, row_len, M, N_alloc, K, out_idx, sentinel, stream, &capturing, &st);
  if (rc != TOPK_OK || st == nullptr) return rc;
  return selector_launch(scores, row_len, M, N_alloc, K, out_idx, sentinel, stream, !capturing, st);
}

int topk_exact_noalloc(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc, int32_t K,
                       int32_t* out_idx, int32_t sentinel, hipStream_t stream) {
  g_err[0] = '\0';
  int rc = selector_args(scores, row_len, M, N_alloc, K, out_idx, sentinel);
  if (rc != TOPK_OK || M == 0) return rc;
  DevState* st = nullptr;
  rc = noalloc_state(&st);
  if (rc != TOPK_OK) return rc;
  return selector_launch(scores, row_len, M, N_alloc, K, out_idx, sentinel, stream, false, st);
}

int topk_exact_sorted(const float* scores, const int32_t* row_len, int64_t M, int64_t N_alloc, int32_t K,
                      int32_t* out_idx, float* out_val, int32_t sentinel, hipStream_t stream) {
  g_err[0] = '\0';
  bool capturing = false;
  DevState* st = nullptr;
  int rc = selector_check(scores, row_len, M, N_alloc, K, out_idx, sentinel, stream, &capturing, &st);
  if (rc != TOPK_OK || st == nullptr) return rc;
  if ((reinterpret_cast<uintptr_t>(out_val) & 3u) != 0) return fail(TOPK_ERR_BAD_ARG, "out_val is not 4-byte aligned");
  // With values wanted, the selector also writes each selected key into out_val (same
  // slot as its index); the sort then reads those instead of gathering the scores again.
  bool sorted_here = false;
  rc = selector_launch(scores, row_len, M, N_alloc, K, out_idx, sentinel, stream, !capturing, st,
                       reinterpret_cast<uint32_t*>(out_val), &sorted_here);
  if (rc != TOPK_OK || sorted_here) return rc;
  // Entries per thread: the smallest power of two with EPT * BLOCK >= K (K <= 4096).
  const dim3 grid((unsigned)M), block(BLOCK);
  const uint32_t NN = (uint32_t)N_alloc, KK = (uint32_t)K;
  if (K <= BLOCK)
    hipLaunchKernelGGL(sort_rows_kernel<1>, grid, block, 0, stream, scores, row_len, NN, KK, out_idx, out_val, sentinel);
  else if (K <= 2 * BLOCK)
    hipLaunchKernelGGL(sort_rows_kernel<2>, grid, block, 0, stream, scores, row_len, NN, KK, out_idx, out_val, sentinel);
  else if (K <= 4 * BLOCK)
    hipLaunchKernelGGL(sort_rows_kernel<4>, grid, block, 0, stream, scores, row_len, NN, KK, out_idx, out_val, sentinel);
  else
    hipLaunchKernelGGL(sort_rows_kernel<8>, grid, block, 0, stream, scores, row_len, NN, KK, out_idx, out_val, sentinel);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch sort_rows_kernel");
  return TOPK_OK;
}

int topk_indexer_topk(const uint8_t* q, const uint8_t* k, const float* w, const int32_t* row_len,
                      int64_t T, int64_t S, int32_t H, int32_t D, int32_t K, float* scores,
                      int32_t* out_idx, int32_t sentinel, hipStream_t stream) {
  g_err[0] = '\0';
  int rc = topk_indexer_check(q, k, w, row_len, T, S, H, D, scores);
  if (rc != TOPK_OK) return rc;
  bool capturing = false;
  DevState* st = nullptr;
  rc = selector_check(scores, row_len, T, S, K, out_idx, sentinel, stream, &capturing, &st);
  if (rc != TOPK_OK || st == nullptr) return rc;
  rc = topk_indexer_launch(q, k, w, row_len, T, S, H, scores, stream);
  if (rc != TOPK_OK) return rc;
  return selector_launch(scores, row_len, T, S, K, out_idx, sentinel, stream, !capturing, st);
}

int topk_exact_reserve(int64_t M_max, int64_t N_alloc_max, int32_t K) {
  g_err[0] = '\0';
  if (M_max < 0 || N_alloc_max < 1 || N_alloc_max > INT32_MAX)
    return fail(TOPK_ERR_BAD_SHAPE, "bad reserve shape");
  if (K < 1 || K > TOPK_K_MAX) return fail(TOPK_ERR_BAD_K, "K = %d outside [1, %d]", K, TOPK_K_MAX);
  DevState* st = nullptr;
  int rc = get_state(false, &st);
  if (rc != TOPK_OK) return rc;
  (void)M_max;  // the workspace does not depend on the call shape
  return TOPK_OK;
}

int topk_exact_get_stats(uint64_t* host_counts, int n, hipStream_t stream) {
  g_err[0] = '\0';
  if (!host_counts) return fail(TOPK_ERR_NULL_POINTER, "host_counts is null");
  if (n < 0 || n > TOPK_STAT_COUNT) return fail(TOPK_ERR_BAD_ARG, "n = %d outside [0, %d]", n, TOPK_STAT_COUNT);
  bool capturing = false;
  int rc = stream_capturing(stream, &capturing);
  if (rc != TOPK_OK) return rc;
  if (capturing) return fail(TOPK_ERR_BAD_ARG, "topk_exact_get_stats cannot run under capture");
  DevState* st = nullptr;
  rc = get_state(false, &st);
  if (rc != TOPK_OK) return rc;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  unsigned long long tmp[TOPK_STAT_COUNT];
  e = hipMemcpy(tmp, st->ctl->stats, sizeof(tmp), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(stats)");
  for (int i = 0; i < n; ++i) host_counts[i] = tmp[i];
  return TOPK_OK;
}

int topk_exact_reset_stats(hipStream_t stream) {
  g_err[0] = '\0';
  bool capturing = false;
  int rc = stream_capturing(stream, &capturing);
  if (rc != TOPK_OK) return rc;
  DevState* st = nullptr;
  rc = get_state(capturing, &st);
  if (rc != TOPK_OK) return rc;
  hipLaunchKernelGGL(zero_stats_kernel, dim3(1), dim3(64), 0, stream, st->ctl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch zero_stats_kernel");
  return TOPK_OK;
}

int topk_exact_set_path_override(int mode) {
  g_err[0] = '\0';
  if (mode < TOPK_PATH_AUTO || mode > TOPK_PATH_RECOVERY)
    return fail(TOPK_ERR_BAD_ARG, "path mode %d unknown", mode);
  g_mode.store(mode);
  return TOPK_OK;
}

int topk_exact_set_execution(int mode) {
  g_err[0] = '\0';
  if (mode < TOPK_EXEC_AUTO || mode > TOPK_EXEC_ROWSPLIT)
    return fail(TOPK_ERR_BAD_ARG, "execution mode %d unknown", mode);
  g_exec.store(mode);
  return TOPK_OK;
}

int topk_exact_time_next_call(hipEvent_t start, hipEvent_t stop) {
  g_err[0] = '\0';
  if ((start == nullptr) != (stop == nullptr))
    return fail(TOPK_ERR_NULL_POINTER, "start and stop must both be set or both be null");
  g_time_start = start;
  g_time_stop = stop;
  return TOPK_OK;
}

int topk_exact_set_proposal(int32_t stride, int32_t rho0_permille, int32_t rho1_permille) {
  g_err[0] = '\0';
  if (stride == 0 && rho0_permille == 0 && rho1_permille == 0) {
    stride = (int32_t)STRIDE;
    rho0_permille = 1500;
    rho1_permille = 1750;
  }
  if (stride < 1 || stride > 65536) return fail(TOPK_ERR_BAD_ARG, "stride %d outside [1, 65536]", stride);
  if (rho0_permille < 500 || rho1_permille < rho0_permille || rho1_permille > 4000)
    return fail(TOPK_ERR_BAD_ARG, "targets %d, %d (thousandths of K) need 500 <= rho0 <= rho1 <= 4000",
                rho0_permille, rho1_permille);
  g_stride.store(stride);
  g_rho0.store(rho0_permille);
  g_rho1.store(rho1_permille);
  return TOPK_OK;
}

int topk_exact_set_admission(int32_t rhoa_permille) {
  g_err[0] = '\0';
  if (rhoa_permille == -1) rhoa_permille = 2250;
  if (rhoa_permille != 0 && (rhoa_permille < 1000 || rhoa_permille > 8000))
    return fail(TOPK_ERR_BAD_ARG, "admission target %d (thousandths of K) needs -1, 0 or 1000..8000", rhoa_permille);
  g_rhoa.store(rhoa_permille);
  return TOPK_OK;
}

int topk_exact_record_phases(uint64_t* buf, int64_t rows, int64_t* wall_clock_khz) {
  g_err[0] = '\0';
  if ((buf == nullptr) != (rows == 0) || rows < 0)
    return fail(TOPK_ERR_BAD_ARG, "buf and rows: both set (rows > 0) or both empty");
  if (wall_clock_khz != nullptr) {
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(wall clock rate)");
    *wall_clock_khz = khz;
  }
  g_phase_rows.store(0);
  g_phase_buf.store(reinterpret_cast<unsigned long long*>(buf));
  g_phase_rows.store(rows);
  return TOPK_OK;
}

const char* topk_exact_last_error(void) { return g_err; }

int topk_stream_read_probe(const float* x, int64_t n, float* sink, hipStream_t stream) {
  g_err[0] = '\0';
  if (n < 0) return fail(TOPK_ERR_BAD_SHAPE, "n = %lld is negative", (long long)n);
  if (n == 0) return TOPK_OK;
  if (!x || !sink) return fail(TOPK_ERR_NULL_POINTER, "null x/sink");
  if ((reinterpret_cast<uintptr_t>(x) & 15u) != 0) return fail(TOPK_ERR_BAD_ARG, "x must be 16-byte aligned");
  bool capturing = false;
  int rc = stream_capturing(stream, &capturing);
  if (rc != TOPK_OK) return rc;
  DevState* st = nullptr;
  rc = get_state(capturing, &st);
  if (rc != TOPK_OK) return rc;
  // One workgroup per 4 MiB chunk (at least one, for the tail elements).
  const int64_t chunks = (n / 4 + (int64_t)PROBE_CHUNK - 1) / (int64_t)PROBE_CHUNK;
  if (chunks > (int64_t)INT32_MAX) return fail(TOPK_ERR_BAD_SHAPE, "n = %lld is too large", (long long)n);
  const unsigned grid = (unsigned)(chunks < 1 ? 1 : chunks);
  hipLaunchKernelGGL(stream_read_probe_kernel, dim3(grid), dim3(BLOCK), 0, stream, x, (uint64_t)n, sink);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "launch stream_read_probe_kernel");
  return TOPK_OK;
}

}  // extern "C"
