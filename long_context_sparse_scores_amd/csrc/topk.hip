// Exact top-k selection on gfx950: radix select over order-preserving keys.
//
// [TEARDOWN, 刀一 DSA] (clawlihai.cn GLM-5.2 1M architecture teardown):
// index_topk 2048 — each query keeps the 2048 best-scoring visible tokens.
// Candidates are s in [0, p]; ties at the threshold go to the lower
// position; the kept positions are written in ascending order, -1 padded.
//
// Scores become uint32 keys whose unsigned order is the float order.  The
// k-th largest key K* is found digit by digit (11 + 11 + 10 bits, most
// significant first).  Each row is cut into slices (a few hundred workgroups
// over all rows, so a few long rows still fill the chip); a slice is cut
// into one contiguous range per wave.  The passes:
//   init    zero the row's global histogram and counters;
//   hist    histogram of the top digit (LDS per slice, non-zero bins added
//           to the row's histogram);
//   filter  every slice finds the threshold digit T from that histogram and
//           appends every key whose top digit is T or above to the row's
//           candidate list (fewer than k lie above T, so the list is the
//           top-k plus the keys that share T's bin);
//   select  one workgroup per row, from the candidates alone: the middle
//           digit of K*; then, when at most 64 keys share K*'s top 22 bits
//           (the usual case), one wave ranks them by key and position;
//           otherwise the low digit, the number of keys equal to K* to take
//           and, when ties straddle the cut, the lowest positions among them
//           (a second radix select, on the complemented position, or a direct
//           ranking of at most 64); the k kept positions are compacted into
//           LDS and written out in ascending order from a bitmap of the row's
//           positions (393216 per chunk, in the space the candidate copy used).
// In the layer group the decode indexer does the first two: it clears the
// counters and adds the top-digit histogram of the scores it holds in
// registers.  That histogram must start from zero, and no launch of the group
// can clear it before the indexer adds to it; so the selection, its last
// user, clears it for the next call and leaves a stamp of the row and the
// shape.  The histogram is used only when that stamp is there and the counts
// add up to the row's visible keys; otherwise (a workspace's first use, or the
// first after a change of shape) the row is counted again from its scores,
// slower but with the same result.
// Filter and select then run as one launch (also for standalone calls of up
// to 256 rows, after the histogram pass): each slice workgroup writes its
// candidates in position order to a region of its own, through to memory, and
// the last one of the row to arrive selects from all regions, so the kept
// positions come out of one ordered compaction with no sort (see
// topk_fused_kernel).  Many rows without the indexer's histogram (prefill)
// keep the separate filter and select launches, whose small filter
// workgroups stream long rows with more of them resident per CU.
// When a row's candidates overflow what the selection can hold (heavily tied
// scores), it scans the whole row instead; the result is the same.
#include "common.h"

namespace dsa {
namespace {

constexpr int kThreads = 256;
constexpr int kSelectThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = kTopBins;
constexpr int kTargetBlocks = 512;   // slices over all rows
constexpr int kMinSlice = 4096;
constexpr int kMaxSlices = 512;      // per row
constexpr int kStage = 256;          // per-wave LDS staging of candidates
constexpr int kBatch = 32;           // loads in flight per lane in the streaming passes
constexpr int kFineSlice = 65536;    // slices at least this long take the 8192-bin LDS histogram
constexpr int kSelMax = 2048;        // the kept positions (k <= 2048) are compacted in LDS
constexpr int kCandLds = 12288;      // candidates the selection holds in LDS
constexpr int kSelBatch = kCandLds / kSelectThreads;  // loads in flight per thread in its passes
constexpr int kFusedTarget = 256;    // slice workgroups over all rows in the fused pass (one per CU)
constexpr int kFusedMaxSlices = 256; // slices per row in the fused pass (count words per row)
constexpr int kFPer = 16;            // keys per thread and batch in the fused pass
constexpr int kFusedMinSlice = kFPer * kSelectThreads;

// Per-row workspace (32-bit words).
// kStT, kStAbove: the threshold digit T and the count of keys whose top digit is above it.
// kCtrDone: the fused pass's slice workgroups that have published their candidates.
// kStamp: written by the selection once it has cleared the row's histogram
// (see histogram_stamp); the counters before it are cleared for every call.
enum : int { kCtrCand = 0, kStT = 1, kStAbove = 2, kCtrDone = 3, kStamp = 7, kCtrWords = 8 };

struct Layout {
    int rows;     // rows (queries) of the call
    int L;        // keys per row
    int slice;    // elements per slice (multiple of 256)
    int nslice;   // slices per row
    int cap;      // candidate capacity per row
    int fslice;   // fused pass: elements per slice (multiple of kSelectThreads)
    int fnslice;  // fused pass: slices per row
    int pcap;     // fused pass: candidate capacity per slice (cap / fnslice)
    __host__ __device__ size_t row_words() const { return kBins + kCtrWords + kFusedMaxSlices + 2 * (size_t)cap; }
};

struct RowWs {
    uint32_t* hist1;   // [kBins] top digit
    uint32_t* ctr;     // [kCtrWords]
    uint32_t* scnt;    // [kFusedMaxSlices] fused pass: candidates per slice
    uint32_t* cpos;    // [cap] candidate positions (fused pass: pcap per slice, in position order)
    uint32_t* ckey;    // [cap] candidate keys
};

__device__ __forceinline__ RowWs row_ws(void* ws, int row, const Layout& lo) {
    uint32_t* b = reinterpret_cast<uint32_t*>(ws) + (size_t)row * lo.row_words();
    RowWs r;
    r.hist1 = b;
    r.ctr = b + kBins;
    r.scnt = r.ctr + kCtrWords;
    r.cpos = r.scnt + kFusedMaxSlices;
    r.ckey = r.cpos + lo.cap;
    return r;
}

// The mark a selection leaves on a row whose histogram it has cleared: a hash
// of the row and of everything that places the row's words in the workspace,
// never 0.  A later call of the same shape that finds it (and a histogram that
// counts the row's visible keys exactly) can trust the histogram its indexer
// added; after a change of shape, or in a workspace never used before, the
// mark does not match and the filter counts the row itself.
__device__ __forceinline__ uint32_t histogram_stamp(const Layout& lo, int row) {
    uint64_t x = ((uint64_t)(uint32_t)lo.rows << 32) ^ (uint64_t)(uint32_t)lo.L;
    x ^= ((uint64_t)lo.row_words() << 20) ^ ((uint64_t)(uint32_t)row * 0x9E3779B97F4A7C15ull);
    x ^= x >> 31;
    x *= 0xBF58476D1CE4E5B9ull;  // SplitMix64 finaliser (Steele, Lea & Flood 2014)
    x ^= x >> 29;
    return (uint32_t)x | 1u;
}

__device__ __forceinline__ int64_t n_visible(const int32_t* q_pos, int row, int L) {
    int64_t p = q_pos[row];
    if (p < 0) return 0;
    return (p < L - 1 ? p : (int64_t)L - 1) + 1;
}

// Rank of this lane among the set lanes of `mask` below it.
__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Workgroup barrier for LDS hand-offs that leaves outstanding global loads in
// flight (__syncthreads would wait for them as well).
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Exclusive prefix sum over a workgroup of NT threads; `scratch` holds NT/64 words of LDS.
template <int NT>
__device__ __forceinline__ uint32_t excl_scan(uint32_t x, uint32_t* scratch, uint32_t* total) {
    constexpr int NW = NT / kWave;
    const int w = threadIdx.x / kWave;
    const uint32_t inc = wave_incl_scan(x);
    if (lane_id() == kWave - 1) scratch[w] = inc;
    lds_sync();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const uint32_t v = scratch[i];
        before += (i < w) ? v : 0u;
        tot += v;
    }
    lds_sync();
    *total = tot;
    return before + inc - x;
}

// This thread's bins of a histogram of `nbins` (<= 2048) bins, highest first:
// thread t holds bins nbins-1 - (per*t + i).
template <int NT>
struct HistPart {
    uint32_t h[kBins / NT];
};

template <int NT>
__device__ __forceinline__ HistPart<NT> load_hist(const uint32_t* hist, int nbins) {
    constexpr int per = kBins / NT;
    HistPart<NT> hp;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        const int bin = nbins - 1 - (per * (int)threadIdx.x + i);
        hp.h[i] = bin >= 0 ? hist[bin] : 0u;
    }
    return hp;
}

// The bin holding the `need`-th largest element (1 <= need <= total), the
// count of elements in higher bins and the count in that bin.  All NT threads call it.
struct BinPick {
    uint32_t bin, above, count;
};

template <int NT>
__device__ __forceinline__ BinPick pick_bin(const HistPart<NT>& hp, int nbins, uint32_t need, uint32_t* scratch,
                                            BinPick* result, uint32_t* total_out = nullptr) {
    constexpr int per = kBins / NT;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) s += hp.h[i];
    if (threadIdx.x == 0) *result = BinPick{0u, 0u, 0u};
    uint32_t total;
    const uint32_t above = excl_scan<NT>(s, scratch, &total);  // count in higher bins (also orders the reset)
    if (total_out) *total_out = total;
    if (above < need && need <= above + s) {
        uint32_t acc = above;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (acc + hp.h[i] >= need) {
                *result = BinPick{(uint32_t)(nbins - 1 - (per * (int)threadIdx.x + i)), acc, hp.h[i]};
                break;
            }
            acc += hp.h[i];
        }
    }
    lds_sync();
    const BinPick r = *result;
    lds_sync();
    return r;
}

// LDS of the selection.  Once the kept positions are compacted, the candidate
// copy's space holds the position bitmap and its per-word prefix counts.
template <int NT>
struct SelectLds {
    union {
        struct {
            uint32_t pos[kCandLds], key[kCandLds];
        } cand;  // copy of the candidate list
        struct {
            uint32_t bits[kCandLds + NT];  // kCandLds * 32 positions per chunk, word w at w + w / (kCandLds / NT)
            uint32_t wpre[kCandLds + NT];  // kept positions in the bitmap words before each word (same layout)
        } order;
    };
    uint32_t h[kBins];
    uint32_t sel[kSelMax];
    uint32_t scratch[NT / kWave];
    uint32_t sbase[kFusedMaxSlices], scnt[kFusedMaxSlices];  // fused pass: slice offsets and counts
    uint32_t sextra[kFusedMaxSlices];                         // fused pass: offsets of entries past the first read
    uint32_t gkey[kWave];                                     // a small group's keys (positions in sel)
    BinPick pick;
    uint32_t nsel, cut, cut_key;
};

// Clear h[0, nbins), let fill(h) add to it, then pick the bin of the need-th largest.
template <int NT, typename Fill>
__device__ __forceinline__ BinPick hist_pick(SelectLds<NT>& s, int nbins, uint32_t need, Fill&& fill) {
    for (int i = threadIdx.x; i < nbins; i += NT) s.h[i] = 0u;
    lds_sync();
    fill(s.h);
    lds_sync();
    const HistPart<NT> hp = load_hist<NT>(s.h, nbins);
    return pick_bin<NT>(hp, nbins, need, s.scratch, &s.pick);
}

// Ordered compaction of one batch over the workgroup: item j of thread t is
// item j*NT + t of the batch (so wave w holds items j*NT + 64w .. +63); every
// flagged item gets emit(slot, j), the slots numbered 0, 1, .. in item order.
// `cnt` holds PER * NT / 64 words of LDS.  Returns the batch's flagged count.
template <int NT, int PER, typename Emit>
__device__ __forceinline__ uint32_t ordered_slots(const bool (&f)[PER], uint32_t* cnt, uint32_t* scratch, Emit&& emit) {
    constexpr int NW = NT / kWave;
    static_assert(PER * NW <= NT, "one count per thread in the scan");
    const int wave = threadIdx.x / kWave;
    uint64_t m[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) m[j] = __ballot(f[j]);
    if (lane_id() == 0) {
#pragma unroll
        for (int j = 0; j < PER; ++j) cnt[j * NW + wave] = (uint32_t)__popcll(m[j]);
    }
    lds_sync();
    const uint32_t x = (int)threadIdx.x < PER * NW ? cnt[threadIdx.x] : 0u;
    uint32_t total;
    const uint32_t ex = excl_scan<NT>(x, scratch, &total);
    if ((int)threadIdx.x < PER * NW) cnt[threadIdx.x] = ex;
    lds_sync();
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (f[j]) emit(cnt[j * NW + wave] + lane_rank(m[j]), j);
    lds_sync();  // before cnt is reused
    return total;
}

// The row's threshold digit T (and the count of keys above its bin) from the
// top-digit histogram in the workspace.  checked: the indexer added that
// histogram onto what the last selection left, so it is used only when that
// selection's stamp is there and it counts the row's visible keys exactly;
// otherwise (a workspace's first use, or the first after a change of shape)
// the row is counted here into own_hist (kBins words of LDS), from its scores.
// hp and stamp: this thread's part of the workspace histogram and the row's
// stamp word, loaded by the caller (with its other first loads).
template <int NT>
__device__ __forceinline__ BinPick row_threshold(const HistPart<NT>& hp, uint32_t stamp,
                                                 const float* __restrict__ row_scores, int64_t n, int k,
                                                 const Layout& lo, int row, bool checked, uint32_t* own_hist,
                                                 uint32_t* scratch, BinPick* pick) {
    uint32_t total;
    BinPick b0 = pick_bin<NT>(hp, kBins, (uint32_t)k, scratch, pick, &total);
    if (checked && (stamp != histogram_stamp(lo, row) || total != (uint32_t)n)) {
        for (int i = threadIdx.x; i < kBins; i += NT) own_hist[i] = 0u;
        lds_sync();
        for (int64_t i = threadIdx.x; i < n; i += NT) atomicAdd(&own_hist[score_key(row_scores[i]) >> 21], 1u);
        lds_sync();
        const HistPart<NT> hp2 = load_hist<NT>(own_hist, kBins);
        b0 = pick_bin<NT>(hp2, kBins, (uint32_t)k, scratch, pick);
    }
    return b0;
}

// The selection is done with the row's histogram (every reader has read it):
// leave it zero for the next selection, whose indexer adds into it, and mark
// it so.
template <int NT>
__device__ __forceinline__ void finish_row(const RowWs& rw, const Layout& lo, int row) {
    for (int i = threadIdx.x; i < kBins; i += NT) rw.hist1[i] = 0u;
    if (threadIdx.x == 0) rw.ctr[kStamp] = histogram_stamp(lo, row);
}

// The last kept key K* and, among the keys equal to it, the highest kept
// position: the kept set is {key > K*} + {key == K*, position <= pos_cut}.
struct Cut {
    uint32_t kstar, pos_cut;
};

// The cut from b1, the bin of K*'s middle digit among the keys whose top digit
// is T (need = k minus the count of keys above T's bin).  for_candidates(f)
// calls f(key, position) for every candidate (every thread takes part).
// Usually few keys share K*'s top 22 bits: then one wave ranks them directly
// (by key, then position); otherwise the low digit and, when ties straddle the
// cut, the positions are radix selected.
template <int NT, typename ForCand>
__device__ __forceinline__ Cut find_cut(SelectLds<NT>& s, uint32_t T, uint32_t need, const BinPick& b1,
                                        ForCand&& for_candidates) {
    const int lane = lane_id();
    const uint32_t need1 = need - b1.above;
    const uint32_t prefix = (T << 11) | b1.bin;  // top 22 bits of K*
    if (b1.count <= (uint32_t)kWave) {
        if (threadIdx.x == 0) s.nsel = 0u;
        lds_sync();
        for_candidates([&](uint32_t key, uint32_t pos) {
            if ((key >> 10) == prefix) {
                const uint32_t slot = atomicAdd(&s.nsel, 1u);
                s.gkey[slot] = key;
                s.sel[slot] = pos;
            }
        });
        lds_sync();
        if (threadIdx.x < kWave) {
            const bool have = (uint32_t)lane < b1.count;
            const uint32_t mk = have ? s.gkey[lane] : 0u, mp = have ? s.sel[lane] : 0xFFFFFFFFu;
            uint32_t rank = 0;  // group members before this one: larger key, or equal key and lower position
            for (uint32_t j = 0; j < b1.count; ++j) {
                const uint32_t ok = s.gkey[j], op = s.sel[j];
                rank += (ok > mk || (ok == mk && op < mp)) ? 1u : 0u;
            }
            if (have && rank == need1 - 1u) {
                s.cut_key = mk;
                s.cut = mp;
            }
        }
        lds_sync();
        const Cut c{s.cut_key, s.cut};
        lds_sync();
        return c;
    }
    const BinPick b2 = hist_pick<NT>(s, 1024, need1, [&](uint32_t* h) {
        for_candidates([&](uint32_t key, uint32_t) {
            if ((key >> 10) == prefix) atomicAdd(&h[key & 0x3FFu], 1u);
        });
    });
    const uint32_t kstar = (prefix << 10) | b2.bin;
    const uint32_t take_eq = need1 - b2.above;  // of the b2.count keys equal to K*
    // ties kept: position <= pos_cut.  When only some are taken, the take_eq
    // lowest positions are the take_eq largest values of ~position (distinct).
    uint32_t pos_cut = 0xFFFFFFFFu;
    if (take_eq < b2.count && b2.count <= (uint32_t)kWave) {
        // few ties: gather them, and one wave ranks each by position
        if (threadIdx.x == 0) s.nsel = 0u;
        lds_sync();
        for_candidates([&](uint32_t key, uint32_t pos) {
            if (key == kstar) s.sel[atomicAdd(&s.nsel, 1u)] = pos;
        });
        lds_sync();
        if (threadIdx.x < kWave) {
            const uint32_t my = (uint32_t)lane < b2.count ? s.sel[lane] : 0xFFFFFFFFu;
            uint32_t rank = 0;
            for (uint32_t j = 0; j < b2.count; ++j) rank += s.sel[j] < my ? 1u : 0u;
            if ((uint32_t)lane < b2.count && rank == take_eq - 1u) s.cut = my;
        }
        lds_sync();
        pos_cut = s.cut;
    } else if (take_eq < b2.count) {
        auto ties = [&](auto&& g) {
            for_candidates([&](uint32_t key, uint32_t pos) {
                if (key == kstar) g(~pos);
            });
        };
        const BinPick t0 = hist_pick<NT>(s, kBins, take_eq, [&](uint32_t* h) {
            ties([&](uint32_t v) { atomicAdd(&h[v >> 21], 1u); });
        });
        const uint32_t tneed1 = take_eq - t0.above;
        const BinPick t1 = hist_pick<NT>(s, kBins, tneed1, [&](uint32_t* h) {
            ties([&](uint32_t v) {
                if ((v >> 21) == t0.bin) atomicAdd(&h[(v >> 10) & 0x7FFu], 1u);
            });
        });
        const uint32_t tneed2 = tneed1 - t1.above;
        const uint32_t tprefix = (t0.bin << 11) | t1.bin;
        const BinPick t2 = hist_pick<NT>(s, 1024, tneed2, [&](uint32_t* h) {
            ties([&](uint32_t v) {
                if ((v >> 10) == tprefix) atomicAdd(&h[v & 0x3FFu], 1u);
            });
        });
        pos_cut = ~((tprefix << 10) | t2.bin);
    }
    return Cut{kstar, pos_cut};
}

// The largest s < n with a[s] <= x, for a non-decreasing a with a[0] <= x and
// n <= kFusedMaxSlices: with a the offsets of consecutive regions in their
// concatenation, the region that holds entry x (the last of any empty ones).
__device__ __forceinline__ int last_le(const uint32_t* a, int n, uint32_t x) {
    int s = 0;
#pragma unroll
    for (int step = kFusedMaxSlices / 2; step > 0; step >>= 1)
        if (s + step < n && a[s + step] <= x) s += step;
    return s;
}

// Where the selection finds the row's candidates (the keys whose top digit is
// T or above): the filter pass's list, the fused pass's per-slice regions (none
// overflowed; s.sbase holds their offsets), or the row's scores.
enum class CandSource { kList, kRegions, kScores };
struct Regions {
    int nact = 0;  // regions (active slices)
    int pcap = 0;  // entries per region
};

// The k kept positions of one row with n > k visible keys, ascending, into
// out[0, k): NT threads.  The candidates number ncand; need = k minus the count
// of keys above T's bin.  Regions are read with device-scope loads (other
// workgroups of this launch wrote them).
template <int NT>
__device__ __forceinline__ void select_row(const float* __restrict__ row_scores, int64_t n, int k, const RowWs& rw,
                                           CandSource src, Regions rg, uint32_t ncand, uint32_t T, uint32_t need,
                                           int32_t* __restrict__ out, SelectLds<NT>& s) {
    const bool from_list = src == CandSource::kList;
    const bool in_lds = from_list && ncand <= (uint32_t)kCandLds;
    const int lane = lane_id();
    constexpr uint32_t kStep = kSelBatch * NT;
    if (in_lds) {  // one batch of loads per thread
        static_assert(kCandLds <= kSelBatch * NT, "the LDS copy is one batch");
        uint32_t cp[kSelBatch], ck[kSelBatch];
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const uint32_t i = j * NT + threadIdx.x;
            cp[j] = i < ncand ? rw.cpos[i] : 0u;
            ck[j] = i < ncand ? rw.ckey[i] : 0u;
        }
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const uint32_t i = j * NT + threadIdx.x;
            if (i < ncand) {
                s.cand.pos[i] = cp[j];
                s.cand.key[i] = ck[j];
            }
        }
        lds_sync();
    }
    // Visit every key of the row whose top digit is T or above in batches of
    // kSelBatch per thread, all loads of a batch issued before any is used:
    // g(key[], pos[], ok[]) with ok[j] set for the batch's candidates.  Every
    // lane of a wave takes part in every call.
    auto visit = [&](auto&& g) {
        uint32_t ck[kSelBatch], cp[kSelBatch];
        bool ok[kSelBatch];
        if (in_lds) {
#pragma unroll
            for (int j = 0; j < kSelBatch; ++j) {
                const uint32_t i = j * NT + threadIdx.x;
                ok[j] = i < ncand;
                ck[j] = ok[j] ? s.cand.key[i] : 0u;
                cp[j] = ok[j] ? s.cand.pos[i] : 0u;
            }
            g(ck, cp, ok);
        } else if (from_list) {
            for (uint32_t i0 = 0; i0 < ncand; i0 += kStep) {
#pragma unroll
                for (int j = 0; j < kSelBatch; ++j) {
                    const uint32_t i = i0 + j * NT + threadIdx.x;
                    ok[j] = i < ncand;
                    ck[j] = ok[j] ? rw.ckey[i] : 0u;
                    cp[j] = ok[j] ? rw.cpos[i] : 0u;
                }
                g(ck, cp, ok);
            }
        } else if (src == CandSource::kRegions) {
            const __amdgpu_buffer_rsrc_t pos_r = wt_rsrc(rw.cpos), key_r = wt_rsrc(rw.ckey);
            for (uint32_t i0 = 0; i0 < ncand; i0 += kStep) {
#pragma unroll
                for (int j = 0; j < kSelBatch; ++j) {
                    const uint32_t i = i0 + j * NT + threadIdx.x;
                    ok[j] = i < ncand;
                    const int r = last_le(s.sbase, rg.nact, ok[j] ? i : 0u);
                    const uint32_t off = 4u * ((uint32_t)r * (uint32_t)rg.pcap + (i - s.sbase[r]));
                    ck[j] = ok[j] ? load_dev4u(key_r, off) : 0u;
                    cp[j] = ok[j] ? load_dev4u(pos_r, off) : 0u;
                }
                g(ck, cp, ok);
            }
        } else {
            for (int64_t i0 = 0; i0 < n; i0 += kStep) {
                float sv[kSelBatch];
#pragma unroll
                for (int j = 0; j < kSelBatch; ++j) {
                    const int64_t i = i0 + j * NT + threadIdx.x;
                    sv[j] = i < n ? row_scores[i] : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < kSelBatch; ++j) {
                    const int64_t i = i0 + j * NT + threadIdx.x;
                    ck[j] = score_key(sv[j]);
                    cp[j] = (uint32_t)i;
                    ok[j] = i < n && (ck[j] >> 21) >= T;
                }
                g(ck, cp, ok);
            }
        }
    };
    // f(key, position) for every candidate
    auto for_candidates = [&](auto&& f) {
        visit([&](const uint32_t (&ck)[kSelBatch], const uint32_t (&cp)[kSelBatch], const bool (&ok)[kSelBatch]) {
#pragma unroll
            for (int j = 0; j < kSelBatch; ++j)
                if (ok[j]) f(ck[j], cp[j]);
        });
    };
    // K*: its middle digit among the keys whose top digit is T, then the cut
    const BinPick b1 = hist_pick<NT>(s, kBins, need, [&](uint32_t* h) {
        for_candidates([&](uint32_t key, uint32_t) {
            if ((key >> 21) == T) atomicAdd(&h[(key >> 10) & 0x7FFu], 1u);
        });
    });
    const Cut cut = find_cut<NT>(s, T, need, b1, for_candidates);
    const uint32_t kstar = cut.kstar, pos_cut = cut.pos_cut;
    // compact the k kept positions: per batch, one LDS atomic per wave
    if (threadIdx.x == 0) s.nsel = 0u;
    lds_sync();
    visit([&](const uint32_t (&ck)[kSelBatch], const uint32_t (&cp)[kSelBatch], const bool (&ok)[kSelBatch]) {
        uint64_t m[kSelBatch];
        uint32_t tot = 0;
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            m[j] = __ballot(ok[j] && (ck[j] > kstar || (ck[j] == kstar && cp[j] <= pos_cut)));
            tot += (uint32_t)__popcll(m[j]);
        }
        uint32_t base = 0;
        if (lane == 0 && tot) base = atomicAdd(&s.nsel, tot);
        base = __shfl(base, 0, kWave);
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            if ((m[j] >> lane) & 1u) {
                const uint32_t slot = base + lane_rank(m[j]);
                if (slot < (uint32_t)kSelMax) s.sel[slot] = cp[j];
            }
            base += (uint32_t)__popcll(m[j]);
        }
    });
    lds_sync();
    // ascending order, per chunk of kCandLds * 32 positions (the candidate copy
    // is no longer needed): a bitmap of the kept positions and the prefix count
    // of its words give every kept position its rank
    static_assert(kCandLds % NT == 0, "whole bitmap words per thread");
    constexpr int kPer = kCandLds / NT;
    // Thread t counts and prefixes words kPer t .. kPer t + kPer - 1.  Word w is
    // stored at pw(w) = w + w / kPer, so thread t's words start at (kPer + 1) t:
    // with an odd stride those loops are free of LDS bank conflicts (a stride of
    // 12 words put 8 lanes on every bank they touched).
    static_assert(kPer % 2 == 0, "odd padded stride");
    auto pw = [](int w) { return w + w / kPer; };
    uint32_t base = 0;
    const __amdgpu_buffer_rsrc_t out_wt = wt_rsrc(out);
    for (int64_t c0 = 0; c0 < n; c0 += (int64_t)kCandLds * 32) {
        const int nw = (int)min((int64_t)kCandLds, (n - c0 + 31) / 32);
        for (int i = threadIdx.x; i < pw(nw - 1) + 1; i += NT) s.order.bits[i] = 0u;
        lds_sync();
        for (int j = threadIdx.x; j < k; j += NT) {
            const int64_t p = (int64_t)s.sel[j] - c0;
            if (p >= 0 && p < (int64_t)nw * 32) atomicOr(&s.order.bits[pw((int)(p >> 5))], 1u << (p & 31));
        }
        lds_sync();
        uint32_t wc[kPer], cnt = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int wi = (int)threadIdx.x * kPer + i;
            wc[i] = wi < nw ? (uint32_t)__popc(s.order.bits[pw(wi)]) : 0u;
            cnt += wc[i];
        }
        uint32_t total;
        uint32_t o = excl_scan<NT>(cnt, s.scratch, &total);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            s.order.wpre[pw((int)threadIdx.x * kPer + i)] = o;
            o += wc[i];
        }
        lds_sync();
        for (int j = threadIdx.x; j < k; j += NT) {
            const int64_t p = (int64_t)s.sel[j] - c0;
            if (p >= 0 && p < (int64_t)nw * 32) {
                const int w = pw((int)(p >> 5));
                const uint32_t below = s.order.bits[w] & ((1u << (p & 31)) - 1u);
                store_wt4(out_wt, 4u * (base + s.order.wpre[w] + (uint32_t)__popc(below)), s.sel[j]);
            }
        }
        base += total;
        lds_sync();  // before the next chunk clears the bitmap
    }
}

__global__ __launch_bounds__(kThreads) void topk_init_kernel(void* ws, Layout lo) {
    RowWs rw = row_ws(ws, blockIdx.x, lo);
    for (int i = threadIdx.x; i < kBins + kCtrWords; i += kThreads) rw.hist1[i] = 0u;  // hist1, ctr
}

// The top digit's histogram of one slice.  FINE > 11 counts 2^FINE bins in
// LDS and folds them to the 2048 top-digit bins on the way out: scores cluster
// in few top-digit bins, so the LDS atomics of one instruction collide, and
// finer bins spread them; that pays on long slices (one per row at prefill),
// where the atomics bound the pass.
// VEC (rows of a multiple of 4 keys, so every slice starts 16-byte aligned):
// 16-byte nontemporal loads, 4 keys per lane and load; the quad holding the
// end of the visible keys is read whole (it lies inside the row) and masked.
template <int FINE, bool VEC>
__global__ __launch_bounds__(kThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ q_pos, int L, int k,
                                                             Layout lo, void* ws) {
    constexpr int kFine = 1 << FINE;
    constexpr int kFold = kFine / kBins;
    static_assert(FINE >= 11, "at least the top digit");
    const int row = blockIdx.x / lo.nslice;
    const int slice = blockIdx.x % lo.nslice;
    const int64_t n = n_visible(q_pos, row, L);
    const int64_t start = (int64_t)slice * lo.slice;
    if (n <= k || start >= n) return;
    __shared__ uint32_t h[kFine];
    for (int i = threadIdx.x; i < kFine; i += kThreads) h[i] = 0u;
    const float* src = scores + (int64_t)row * L + start;
    const int m = (int)((n - start) < lo.slice ? (n - start) : lo.slice);
    lds_sync();
    if constexpr (VEC) {
        for (int i0 = 0; i0 < m; i0 += kBatch * kThreads) {
            f32x4_t v[kBatch / 4];
#pragma unroll
            for (int j = 0; j < kBatch / 4; ++j) {
                const int i = i0 + 4 * (j * kThreads + (int)threadIdx.x);
                v[j] = i < m ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(src + i))
                             : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int j = 0; j < kBatch / 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (i0 + 4 * (j * kThreads + (int)threadIdx.x) + e < m)
                        atomicAdd(&h[score_key(v[j][e]) >> (32 - FINE)], 1u);
        }
    } else {
        for (int i0 = 0; i0 < m; i0 += kBatch * kThreads) {
            float v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int i = i0 + j * kThreads + threadIdx.x;
                v[j] = i < m ? src[i] : 0.0f;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (i0 + j * kThreads + (int)threadIdx.x < m) atomicAdd(&h[score_key(v[j]) >> (32 - FINE)], 1u);
        }
    }
    lds_sync();
    uint32_t* g = row_ws(ws, row, lo).hist1;
    for (int i = threadIdx.x; i < kBins; i += kThreads) {
        uint32_t c = 0;
#pragma unroll
        for (int f = 0; f < kFold; ++f) c += h[i * kFold + f];
        if (c) atomicAdd(&g[i], c);
    }
}

// hist_checked: the histogram was added by the indexer onto what the last
// selection left, so it is used only when that selection's stamp is there and
// it counts the row's visible keys exactly; otherwise it was built from zero
// in this call.  VEC: 16-byte nontemporal loads as in topk_hist_kernel (each
// wave's range starts at a multiple of 64 keys); the candidates reach the
// row's list in another order, which the selection does not depend on.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void topk_filter_kernel(const float* __restrict__ scores,
                                                               const int32_t* __restrict__ q_pos, int L, int k,
                                                               Layout lo, void* ws, int hist_checked) {
    const int row = blockIdx.x / lo.nslice;
    const int slice = blockIdx.x % lo.nslice;
    const int64_t n = n_visible(q_pos, row, L);
    const int64_t start = (int64_t)slice * lo.slice;
    if (n <= k || start >= n) return;
    const int lane = lane_id();
    const int wave = threadIdx.x / kWave;
    RowWs rw = row_ws(ws, row, lo);

    __shared__ uint32_t stage_pos[kWaves][kStage], stage_key[kWaves][kStage];
    __shared__ uint32_t scratch[kWaves];
    __shared__ BinPick pick;
    __shared__ uint32_t own_hist[kBins];  // only when the row's histogram cannot be trusted

    // the histogram, the stamp and this wave's first batch of scores in flight together
    const HistPart<kThreads> hp = load_hist<kThreads>(rw.hist1, kBins);
    const uint32_t stamp = rw.ctr[kStamp];
    const int64_t w0 = start + (int64_t)wave * (lo.slice / kWaves);
    const int64_t w1 = min(w0 + lo.slice / kWaves, n);
    const float* row_scores = scores + (int64_t)row * L;
    float v[kBatch];
    // value j of this lane: key i0 + j * 64 + lane, or (VEC) i0 + 4 * ((j / 4) * 64 + lane) + j % 4
    auto key_at = [&](int64_t i0, int j) -> int64_t {
        return VEC ? i0 + 4 * ((j / 4) * kWave + lane) + (j % 4) : i0 + j * kWave + lane;
    };
    auto load_batch = [&](int64_t i0) {
        if constexpr (VEC) {
#pragma unroll
            for (int j = 0; j < kBatch / 4; ++j) {
                const int64_t i = i0 + 4 * (j * kWave + lane);
                // a quad starting before w1 lies inside the row (L is a multiple of 4); past w1 never used
                const f32x4_t x = __builtin_nontemporal_load(
                    reinterpret_cast<const f32x4_t*>(row_scores + (i < w1 ? i : (w1 - 1) / 4 * 4)));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * j + e] = x[e];
            }
        } else {
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int64_t i = i0 + j * kWave + lane;
                v[j] = row_scores[i < w1 ? i : w1 - 1];  // w1 >= 1; past w1 never used
            }
        }
    };
    load_batch(w0);
    const BinPick b0 = row_threshold<kThreads>(hp, stamp, row_scores, n, k, lo, row, hist_checked != 0, own_hist,
                                               scratch, &pick);
    const uint32_t T = b0.bin;
    if (slice == 0 && threadIdx.x == 0) {  // for the selection
        rw.ctr[kStT] = T;
        rw.ctr[kStAbove] = b0.above;
    }

    // Candidates are staged per wave in LDS and appended to the row's list in
    // batches: one global atomic per batch rather than per 64 keys.
    uint32_t staged = 0;  // wave-uniform
    const __amdgpu_buffer_rsrc_t cpos_out = wt_rsrc(rw.cpos), ckey_out = wt_rsrc(rw.ckey);
    uint32_t* sp = stage_pos[wave];
    uint32_t* sk = stage_key[wave];
    auto flush = [&]() {
        __builtin_amdgcn_wave_barrier();
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&rw.ctr[kCtrCand], staged);
        base = __shfl(base, 0, kWave);
        for (uint32_t j = lane; j < staged; j += kWave) {
            const uint32_t slot = base + j;
            if (slot < (uint32_t)lo.cap) {
                store_wt4(cpos_out, 4u * slot, sp[j]);
                store_wt4(ckey_out, 4u * slot, sk[j]);
            }
        }
        __builtin_amdgcn_wave_barrier();
        staged = 0;
    };
    for (int64_t i0 = w0; i0 < w1; i0 += kBatch * kWave) {
        if (i0 != w0) load_batch(i0);
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = key_at(i0, j);
            const uint32_t key = score_key(v[j]);
            const bool cand = i < w1 && (key >> 21) >= T;
            const uint64_t m = __ballot(cand);
            if (m) {
                const uint32_t c = (uint32_t)__popcll(m);
                if (staged + c > (uint32_t)kStage) flush();
                if (cand) {
                    const uint32_t slot = staged + lane_rank(m);
                    sp[slot] = (uint32_t)i;
                    sk[slot] = key;
                }
                staged += c;
            }
        }
    }
    if (staged) flush();
}

// One workgroup per row: the k kept positions in ascending order (rows with
// at most k visible positions: all of them, then -1).
__global__ __launch_bounds__(kSelectThreads) void topk_select_kernel(const float* __restrict__ scores,
                                                                     const int32_t* __restrict__ q_pos, int L,
                                                                     int k, Layout lo, void* ws,
                                                                     int32_t* __restrict__ idx) {
    const int row = blockIdx.x;
    const int64_t n = n_visible(q_pos, row, L);
    int32_t* out = idx + (int64_t)row * k;
    const RowWs rw = row_ws(ws, row, lo);
    finish_row<kSelectThreads>(rw, lo, row);  // the filter pass was the histogram's last reader
    if (n <= k) {
        for (int j = threadIdx.x; j < k; j += kSelectThreads) out[j] = j < n ? j : -1;
        return;
    }
    __shared__ SelectLds<kSelectThreads> sl;
    const uint32_t ncand = rw.ctr[kCtrCand];
    select_row<kSelectThreads>(scores + (int64_t)row * L, n, k, rw,
                               ncand <= (uint32_t)lo.cap ? CandSource::kList : CandSource::kScores, Regions(), ncand,
                               rw.ctr[kStT], (uint32_t)k - rw.ctr[kStAbove], out, sl);
}

// Filter and selection in one launch, for rows whose top-digit histogram the
// indexer added (the layer group).  Each row is cut into slices of whole
// batches (about one workgroup per CU over all rows).  A slice workgroup finds
// T from the histogram, and writes the keys of its slice whose top digit is T
// or above, in position order (a workgroup prefix scan per batch, no global
// atomics), to its own region of pcap entries, then its count; those stores
// go through to memory and are acknowledged before the workgroup counts its
// arrival.  The last slice workgroup of the row to arrive selects: it reads
// the counts and the regions with device-scope loads (they were written on
// other XCDs in this launch), so the candidates land in LDS in position
// order, re-reads the scores of any slice whose region overflowed, finds the
// cut, and writes the kept positions through one ordered compaction, already
// ascending.  No workgroup waits for another.  More candidates than the LDS
// copy holds: the selection scans the row's scores (same result, slower).
__global__ __launch_bounds__(kSelectThreads) void topk_fused_kernel(const float* __restrict__ scores,
                                                                    const int32_t* __restrict__ q_pos, int L, int k,
                                                                    Layout lo, void* ws, int hist_checked,
                                                                    int32_t* __restrict__ idx) {
    constexpr int NT = kSelectThreads;
    const int row = blockIdx.x / lo.fnslice;
    const int slice = blockIdx.x % lo.fnslice;
    const RowWs rw = row_ws(ws, row, lo);
    int32_t* out = idx + (int64_t)row * k;
    __shared__ SelectLds<NT> sl;
    const float* row_scores = scores + (int64_t)row * L;
    const int64_t start = (int64_t)slice * lo.fslice;
    const int64_t lim = min(start + (int64_t)lo.fslice, (int64_t)L);  // the slice within the row
    float v[kFPer];
    auto load_batch = [&](int64_t i0, int64_t i1) {  // i0 < i1; past i1 a valid key is read, never used
#pragma unroll
        for (int j = 0; j < kFPer; ++j) {
            const int64_t i = i0 + j * NT + threadIdx.x;
            v[j] = row_scores[i < i1 ? i : i1 - 1];
        }
    };
    // Every first load in one round trip: the row's length, the histogram and
    // its stamp, and this thread's first batch of the slice (up to the row's
    // end; keys past the visible ones are masked below).  The threshold comes
    // before any branch on the length, so no load waits for it.  (Rows with
    // n <= k get a meaningless threshold, unused.)
    const int64_t n = n_visible(q_pos, row, L);
    const HistPart<NT> hp = load_hist<NT>(rw.hist1, kBins);
    const uint32_t stamp = rw.ctr[kStamp];
    load_batch(start, lim);
    const BinPick b0 =
        row_threshold<NT>(hp, stamp, row_scores, n, k, lo, row, hist_checked != 0, sl.h, sl.scratch, &sl.pick);
    const uint32_t T = b0.bin;
    if (n <= k) {
        if (slice == 0) {
            finish_row<NT>(rw, lo, row);
            for (int j = threadIdx.x; j < k; j += NT) out[j] = j < n ? j : -1;
        }
        return;
    }
    if (start >= n) return;  // not counted: the row has nact active slices
    const int64_t end = min(lim, n);
    const int nact = (int)((n + lo.fslice - 1) / lo.fslice);

    // This slice's candidates, in position order, to its region.
    {
        const __amdgpu_buffer_rsrc_t pos_r = wt_rsrc(rw.cpos + (int64_t)slice * lo.pcap);
        const __amdgpu_buffer_rsrc_t key_r = wt_rsrc(rw.ckey + (int64_t)slice * lo.pcap);
        uint32_t run = 0;
        for (int64_t i0 = start; i0 < end; i0 += (int64_t)kFPer * NT) {
            if (i0 != start) load_batch(i0, end);
            bool f[kFPer];
            uint32_t key[kFPer];
#pragma unroll
            for (int j = 0; j < kFPer; ++j) {
                key[j] = score_key(v[j]);
                f[j] = i0 + j * NT + (int)threadIdx.x < end && (key[j] >> 21) >= T;
            }
            const uint32_t c = ordered_slots<NT, kFPer>(f, sl.sel, sl.scratch, [&](uint32_t slot, int j) {
                slot += run;
                if (slot < (uint32_t)lo.pcap) {
                    store_wt4(pos_r, 4u * slot, (uint32_t)(i0 + j * NT + threadIdx.x));
                    store_wt4(key_r, 4u * slot, key[j]);
                }
            });
            run += c;
        }
        if (threadIdx.x == 0) store_wt4(wt_rsrc(rw.scnt), 4u * (uint32_t)slice, run);
    }
    // Publish: the stores above are acknowledged, then the arrival is counted.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
        sl.cut = __hip_atomic_fetch_add(&rw.ctr[kCtrDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u ==
                         (uint32_t)nact
                     ? 1u
                     : 0u;
    __syncthreads();
    if (!sl.cut) return;

    // ---- the last slice workgroup of the row selects
    finish_row<NT>(rw, lo, row);  // every slice has read the histogram
    const uint32_t need = (uint32_t)k - b0.above;
    // The counts and the first W entries of every region in one round trip
    // (W = kCandLds / nact: the regions' usual fill); entries of a region past
    // W are loaded afterwards.
    const __amdgpu_buffer_rsrc_t pos_r = wt_rsrc(rw.cpos), key_r = wt_rsrc(rw.ckey);
    const uint32_t W = (uint32_t)(kCandLds / nact);
    const uint32_t my_cnt = (int)threadIdx.x < nact ? load_dev4u(wt_rsrc(rw.scnt), 4u * threadIdx.x) : 0u;
    uint32_t cp[kSelBatch], ck[kSelBatch];
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) {
        const uint32_t e = j * NT + threadIdx.x;
        const uint32_t sidx = e / W, o = e - sidx * W;
        const bool ok = sidx < (uint32_t)nact && o < (uint32_t)lo.pcap;
        const uint32_t off = 4u * (sidx * (uint32_t)lo.pcap + o);
        cp[j] = ok ? load_dev4u(pos_r, off) : 0u;
        ck[j] = ok ? load_dev4u(key_r, off) : 0u;
    }
    if (threadIdx.x == 0) sl.nsel = 0u;  // bit 0: a region holds more than W entries; bit 1: one overflowed
    uint32_t ncand;
    const uint32_t my_base = excl_scan<NT>(my_cnt, sl.scratch, &ncand);
    if ((int)threadIdx.x < nact) {
        sl.sbase[threadIdx.x] = my_base;
        sl.scnt[threadIdx.x] = my_cnt;
        if (my_cnt > (uint32_t)lo.pcap) atomicOr(&sl.nsel, 2u);
        else if (my_cnt > W) atomicOr(&sl.nsel, 1u);
    }
    for (int i = threadIdx.x; i < kBins; i += NT) sl.h[i] = 0u;
    lds_sync();
    const uint32_t beyond = sl.nsel;
    if (ncand > (uint32_t)kCandLds && (beyond & 2u)) {  // too many to hold, and a region overflowed
        select_row<NT>(row_scores, n, k, rw, CandSource::kScores, Regions(), ncand, T, need, out, sl);
        return;
    }
    BinPick b1;        // the middle digit of K* among the keys in T's bin
    uint32_t nlds;     // candidates in the LDS copy, in position order
    if (ncand > (uint32_t)kCandLds) {
        // More candidates than the LDS copy holds (long rows): one pass over
        // the regions finds the middle digit, a second copies to LDS only the
        // keys whose top 22 bits are K*'s or above, about k of them.
        auto region_batch = [&](uint32_t i0, uint32_t (&ck)[kSelBatch], uint32_t (&cp)[kSelBatch],
                                bool (&ok)[kSelBatch]) {
#pragma unroll
            for (int j = 0; j < kSelBatch; ++j) {
                const uint32_t i = i0 + j * NT + threadIdx.x;
                ok[j] = i < ncand;
                const int r = last_le(sl.sbase, nact, ok[j] ? i : 0u);
                const uint32_t off = 4u * ((uint32_t)r * (uint32_t)lo.pcap + (i - sl.sbase[r]));
                ck[j] = ok[j] ? load_dev4u(key_r, off) : 0u;
                cp[j] = ok[j] ? load_dev4u(pos_r, off) : 0u;
            }
        };
        for (uint32_t i0 = 0; i0 < ncand; i0 += kSelBatch * NT) {
            uint32_t ck[kSelBatch], cq[kSelBatch];
            bool ok[kSelBatch];
            region_batch(i0, ck, cq, ok);
#pragma unroll
            for (int j = 0; j < kSelBatch; ++j)
                if (ok[j] && (ck[j] >> 21) == T) atomicAdd(&sl.h[(ck[j] >> 10) & 0x7FFu], 1u);
        }
        lds_sync();
        b1 = pick_bin<NT>(load_hist<NT>(sl.h, kBins), kBins, need, sl.scratch, &sl.pick);
        const uint32_t prefix = (T << 11) | b1.bin;
        const uint32_t nsel = ((uint32_t)k - need) + b1.above + b1.count;  // keys at K*'s top 22 bits or above
        if (nsel > (uint32_t)kCandLds) {  // so many keys tied on K*'s top 22 bits: passes over the regions
            Regions rg;
            rg.nact = nact;
            rg.pcap = lo.pcap;
            select_row<NT>(row_scores, n, k, rw, CandSource::kRegions, rg, ncand, T, need, out, sl);
            return;
        }
        uint32_t run = 0;
        for (uint32_t i0 = 0; i0 < ncand; i0 += kSelBatch * NT) {
            uint32_t ck[kSelBatch], cq[kSelBatch];
            bool ok[kSelBatch], f[kSelBatch];
            region_batch(i0, ck, cq, ok);
#pragma unroll
            for (int j = 0; j < kSelBatch; ++j) f[j] = ok[j] && (ck[j] >> 10) >= prefix;
            const uint32_t c = ordered_slots<NT, kSelBatch>(f, sl.sel, sl.scratch, [&](uint32_t slot, int j) {
                slot += run;
                if (slot < (uint32_t)kCandLds) {
                    sl.cand.pos[slot] = cq[j];
                    sl.cand.key[slot] = ck[j];
                }
            });
            run += c;
        }
        nlds = run;  // == nsel
    } else {
        // Candidates to LDS in position order (entry o of slice s's region is
        // candidate sbase[s] + o), counting the middle digit of those in T's bin.
        auto place = [&](uint32_t c, uint32_t pos, uint32_t key) {
            sl.cand.pos[c] = pos;
            sl.cand.key[c] = key;
            if ((key >> 21) == T) atomicAdd(&sl.h[(key >> 10) & 0x7FFu], 1u);
        };
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const uint32_t e = j * NT + threadIdx.x;
            const uint32_t sidx = e / W, o = e - sidx * W;
            if (sidx < (uint32_t)nact) {
                const uint32_t cs = sl.scnt[sidx];
                if (o < cs && cs <= (uint32_t)lo.pcap) place(sl.sbase[sidx] + o, cp[j], ck[j]);  // overflowed: below
            }
        }
        if (beyond & 1u) {
            // Entries W.. of the regions that hold more (and did not overflow), in
            // one round: their extra counts, scanned, address them like the regions.
            const uint32_t cs = (int)threadIdx.x < nact ? sl.scnt[threadIdx.x] : 0u;
            uint32_t nextra;
            const uint32_t ex = excl_scan<NT>(cs > W && cs <= (uint32_t)lo.pcap ? cs - W : 0u, sl.scratch, &nextra);
            if ((int)threadIdx.x < nact) sl.sextra[threadIdx.x] = ex;
            lds_sync();
            for (uint32_t i0 = 0; i0 < nextra; i0 += kSelBatch * NT) {
                uint32_t xp[kSelBatch], xk[kSelBatch], xc[kSelBatch];
                bool xo[kSelBatch];
#pragma unroll
                for (int j = 0; j < kSelBatch; ++j) {
                    const uint32_t i = i0 + j * NT + threadIdx.x;
                    xo[j] = i < nextra;
                    const int r = last_le(sl.sextra, nact, xo[j] ? i : 0u);
                    const uint32_t o = W + (i - sl.sextra[r]);
                    const uint32_t off = 4u * ((uint32_t)r * (uint32_t)lo.pcap + o);
                    xc[j] = sl.sbase[r] + o;
                    xp[j] = xo[j] ? load_dev4u(pos_r, off) : 0u;
                    xk[j] = xo[j] ? load_dev4u(key_r, off) : 0u;
                }
#pragma unroll
                for (int j = 0; j < kSelBatch; ++j)
                    if (xo[j]) place(xc[j], xp[j], xk[j]);
            }
        }
        const bool overflowed = (beyond & 2u) != 0u;
        for (int sidx = 0; overflowed && sidx < nact; ++sidx) {
            if (sl.scnt[sidx] <= (uint32_t)lo.pcap) continue;
            // this slice's region overflowed: its candidates again, from its scores
            const int64_t s0 = (int64_t)sidx * lo.fslice, s1 = min(s0 + (int64_t)lo.fslice, n);
            uint32_t run = sl.sbase[sidx];
            for (int64_t i0 = s0; i0 < s1; i0 += (int64_t)kFPer * NT) {
                load_batch(i0, s1);
                bool f[kFPer];
                uint32_t key[kFPer];
#pragma unroll
                for (int j = 0; j < kFPer; ++j) {
                    key[j] = score_key(v[j]);
                    f[j] = i0 + j * NT + (int)threadIdx.x < s1 && (key[j] >> 21) >= T;
                }
                const uint32_t c = ordered_slots<NT, kFPer>(f, sl.sel, sl.scratch, [&](uint32_t slot, int j) {
                    slot += run;  // below ncand: the same scores and T give the same count
                    if (slot < (uint32_t)kCandLds) {
                        sl.cand.pos[slot] = (uint32_t)(i0 + j * NT + threadIdx.x);
                        sl.cand.key[slot] = key[j];
                        if ((key[j] >> 21) == T) atomicAdd(&sl.h[(key[j] >> 10) & 0x7FFu], 1u);
                    }
                });
                run += c;
            }
        }
        lds_sync();
        b1 = pick_bin<NT>(load_hist<NT>(sl.h, kBins), kBins, need, sl.scratch, &sl.pick);
        nlds = ncand;
    }
    auto for_candidates = [&](auto&& f) {
#pragma unroll
        for (int j = 0; j < kSelBatch; ++j) {
            const uint32_t c = j * NT + threadIdx.x;
            if (c < nlds) f(sl.cand.key[c], sl.cand.pos[c]);
        }
    };
    const Cut cut = find_cut<NT>(sl, T, need, b1, for_candidates);
    // the kept candidates, in position order, are the output
    bool f[kSelBatch];
    uint32_t kp[kSelBatch];
#pragma unroll
    for (int j = 0; j < kSelBatch; ++j) {
        const uint32_t c = j * NT + threadIdx.x;
        const uint32_t key = c < nlds ? sl.cand.key[c] : 0u;
        kp[j] = c < nlds ? sl.cand.pos[c] : 0u;
        f[j] = c < nlds && (key > cut.kstar || (key == cut.kstar && kp[j] <= cut.pos_cut));
    }
    const __amdgpu_buffer_rsrc_t out_wt = wt_rsrc(out);
    ordered_slots<NT, kSelBatch>(f, sl.sel, sl.scratch,
                                 [&](uint32_t slot, int j) {
                                     if (slot < (uint32_t)k) store_wt4(out_wt, 4u * slot, kp[j]);  // exactly k kept
                                 });
}


Layout make_layout(int rows, int L) {
    const int max_slices = (L + kMinSlice - 1) / kMinSlice;
    int ns = (kTargetBlocks + rows - 1) / rows;
    if (ns > max_slices) ns = max_slices;
    if (ns > kMaxSlices) ns = kMaxSlices;
    if (ns < 1) ns = 1;
    int64_t slice = ((int64_t)L + ns - 1) / ns;
    slice = (slice + 255) / 256 * 256;
    Layout lo;
    lo.rows = rows;
    lo.L = L;
    lo.slice = (int)slice;
    lo.nslice = (int)(((int64_t)L + slice - 1) / slice);
    int64_t cap = (int64_t)L / 8;
    if (cap < 4096) cap = 4096;
    lo.cap = (int)((cap + 63) / 64 * 64);
    // fused pass: about one slice workgroup per CU over all rows
    int fns = (kFusedTarget + rows - 1) / rows;
    const int fmax = (L + kFusedMinSlice - 1) / kFusedMinSlice;
    if (fns > fmax) fns = fmax;
    if (fns > kFusedMaxSlices) fns = kFusedMaxSlices;
    if (fns < 1) fns = 1;
    int64_t fslice = ((int64_t)L + fns - 1) / fns;
    fslice = (fslice + kSelectThreads - 1) / kSelectThreads * kSelectThreads;
    lo.fslice = (int)fslice;
    lo.fnslice = (int)(((int64_t)L + fslice - 1) / fslice);
    lo.pcap = lo.cap / lo.fnslice;
    return lo;
}

}  // namespace

size_t topk_ws_bytes(int rows, int L, int k) {
    (void)k;
    return align_up((size_t)rows * make_layout(rows, L).row_words() * sizeof(uint32_t), 256);
}

TopkPrep topk_prep(void* ws, int rows, int L, bool hist) {
    const Layout lo = make_layout(rows, L);
    TopkPrep p;
    p.base = reinterpret_cast<uint32_t*>(ws);  // each row's words start with hist1, then the counters
    p.stride = (int64_t)lo.row_words();
    p.zero_off = hist ? kBins : 0;
    p.zero_count = hist ? kStamp : kBins + kStamp;  // the counters before the stamp (and the histogram)
    p.hist = hist;
    return p;
}

hipError_t launch_topk(const float* scores, const int32_t* q_pos, int rows, int L, int k, int32_t* idx, void* ws,
                       hipStream_t stream, TopkState state) {
    const Layout lo = make_layout(rows, L);
    const unsigned grid = (unsigned)((int64_t)rows * lo.nslice);
    // 16-byte loads in the streaming passes when every row starts 16-byte aligned
    const bool vec = L % 4 == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
    if (state == TopkState::kNone) hipLaunchKernelGGL(topk_init_kernel, dim3(rows), dim3(kThreads), 0, stream, ws, lo);
    // finer LDS bins for long slices (measured: prefill 4096 x 128K rows, one slice per row)
    if (state != TopkState::kHistogram)
        hipLaunchKernelGGL(lo.slice >= kFineSlice ? (vec ? topk_hist_kernel<13, true> : topk_hist_kernel<13, false>)
                                                  : (vec ? topk_hist_kernel<11, true> : topk_hist_kernel<11, false>),
                           dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws);
    // The fused pass unless there are many rows (prefill) and no histogram
    // from the indexer: there the separate filter's small workgroups stream
    // the rows with more of them resident per CU.
    if (state == TopkState::kHistogram || rows <= kFusedTarget) {
        hipLaunchKernelGGL(topk_fused_kernel, dim3((unsigned)((int64_t)rows * lo.fnslice)), dim3(kSelectThreads), 0,
                           stream, scores, q_pos, L, k, lo, ws, state == TopkState::kHistogram ? 1 : 0, idx);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(vec ? topk_filter_kernel<true> : topk_filter_kernel<false>, dim3(grid), dim3(kThreads), 0,
                       stream, scores, q_pos, L, k, lo, ws, 0);
    hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(kSelectThreads), 0, stream, scores, q_pos, L, k, lo, ws,
                       idx);
    return hipGetLastError();
}

}  // namespace dsa
