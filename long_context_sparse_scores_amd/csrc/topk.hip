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
//   select  one workgroup per row, from the candidates alone: the middle and
//           low digits of K*, the number of keys equal to K* to take and,
//           when ties straddle the cut, the lowest positions among them (a
//           second radix select, on the complemented position, or a direct
//           ranking when there are at most 64 of them); the k kept positions
//           are compacted into LDS and written out in ascending order from a
//           bitmap of the row's positions (393216 per chunk, in the space the
//           candidate copy used).
// In the layer group the decode indexer does the first two: it clears the
// counters and adds the top-digit histogram of the scores it holds in
// registers, so the scores are read once (filter) and select never touches
// them.  That histogram must start from zero, and no launch of the group can
// clear it before the indexer adds to it; so the selection, its last user,
// clears it for the next call and leaves a stamp of the row and the shape.
// The filter uses the histogram only when it finds that stamp and the counts
// add up to the row's visible keys; otherwise (a workspace's first use, or
// the first after a change of shape) it counts the row itself, slower but
// with the same result.
// (Running select in the last filter workgroup of each row would save a
// launch, but publishing the candidates across XCDs then takes an L2
// write-back per workgroup, which costs far more on this part.)
// When a row's candidate list overflows its capacity (heavily tied scores),
// select scans the whole row instead; the result is the same.
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

// Per-row workspace (32-bit words).
// kStT, kStAbove: the threshold digit T and the count of keys whose top digit is above it.
// kStamp: written by the selection once it has cleared the row's histogram
// (see histogram_stamp); the counters before it are cleared for every call.
enum : int { kCtrCand = 0, kStT = 1, kStAbove = 2, kStamp = 7, kCtrWords = 8 };

struct Layout {
    int rows;     // rows (queries) of the call
    int L;        // keys per row
    int slice;    // elements per slice (multiple of 256)
    int nslice;   // slices per row
    int cap;      // candidate capacity per row
    __host__ __device__ size_t row_words() const { return kBins + kCtrWords + 2 * (size_t)cap; }
};

struct RowWs {
    uint32_t* hist1;   // [kBins] top digit
    uint32_t* ctr;     // [kCtrWords]
    uint32_t* cpos;    // [cap] candidate positions
    uint32_t* ckey;    // [cap] candidate keys
};

__device__ __forceinline__ RowWs row_ws(void* ws, int row, const Layout& lo) {
    uint32_t* b = reinterpret_cast<uint32_t*>(ws) + (size_t)row * lo.row_words();
    RowWs r;
    r.hist1 = b;
    r.ctr = b + kBins;
    r.cpos = r.ctr + kCtrWords;
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
    BinPick pick;
    uint32_t nsel, cut;
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

// The k kept positions of one row with n > k visible keys, ascending, into
// out[0, k): NT threads, the candidate list (keys with top digit >= T) of the
// filter pass, or the row's scores after an overflow.
template <int NT>
__device__ __forceinline__ void select_row(const float* __restrict__ row_scores, int64_t n, int k, const RowWs& rw,
                                           int cap, int32_t* __restrict__ out, SelectLds<NT>& s) {
    const uint32_t ncand = rw.ctr[kCtrCand];
    const uint32_t T = rw.ctr[kStT];
    const uint32_t need = (uint32_t)k - rw.ctr[kStAbove];
    const bool from_list = ncand <= (uint32_t)cap;                  // else the list overflowed
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
    // K*: its middle and low digits among the keys whose top digit is T
    const BinPick b1 = hist_pick<NT>(s, kBins, need, [&](uint32_t* h) {
        for_candidates([&](uint32_t key, uint32_t) {
            if ((key >> 21) == T) atomicAdd(&h[(key >> 10) & 0x7FFu], 1u);
        });
    });
    const uint32_t need1 = need - b1.above;
    const uint32_t prefix = (T << 11) | b1.bin;  // top 22 bits of K*
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
template <int FINE>
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
// in this call.
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

    // the row's top-digit histogram, then this wave's first batch of scores
    const HistPart<kThreads> hp = load_hist<kThreads>(rw.hist1, kBins);
    const int64_t w0 = start + (int64_t)wave * (lo.slice / kWaves);
    const int64_t w1 = min(w0 + lo.slice / kWaves, n);
    const float* row_scores = scores + (int64_t)row * L;
    float v[kBatch];
    auto load_batch = [&](int64_t i0) {
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int64_t i = i0 + j * kWave + lane;
            v[j] = i < w1 ? row_scores[i] : 0.0f;
        }
    };
    load_batch(w0);
    uint32_t total;
    BinPick b0 = pick_bin<kThreads>(hp, kBins, (uint32_t)k, scratch, &pick, &total);
    if (hist_checked && (rw.ctr[kStamp] != histogram_stamp(lo, row) || total != (uint32_t)n)) {
        // The histogram did not start from zero: no selection of this shape
        // cleared it before the indexer added to it (a workspace's first use, or
        // the first after a change of shape).  Count this row here, from its scores.
        for (int i = threadIdx.x; i < kBins; i += kThreads) own_hist[i] = 0u;
        lds_sync();
        for (int64_t i = threadIdx.x; i < n; i += kThreads) atomicAdd(&own_hist[score_key(row_scores[i]) >> 21], 1u);
        lds_sync();
        const HistPart<kThreads> hp2 = load_hist<kThreads>(own_hist, kBins);
        b0 = pick_bin<kThreads>(hp2, kBins, (uint32_t)k, scratch, &pick);
    }
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
            const int64_t i = i0 + j * kWave + lane;
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
                                                                     int32_t* __restrict__ idx, RowClear clear) {
    const int row = blockIdx.x;
    if (clear.base)
        for (int i = threadIdx.x; i < clear.words; i += kSelectThreads) clear.base[(int64_t)row * clear.words + i] = 0u;
    const int64_t n = n_visible(q_pos, row, L);
    int32_t* out = idx + (int64_t)row * k;
    const RowWs rw = row_ws(ws, row, lo);
    // The filter pass was the histogram's last reader: leave it zero for the
    // next selection, whose indexer adds into it, and mark it so.
    for (int i = threadIdx.x; i < kBins; i += kSelectThreads) rw.hist1[i] = 0u;
    if (threadIdx.x == 0) rw.ctr[kStamp] = histogram_stamp(lo, row);
    if (n <= k) {
        for (int j = threadIdx.x; j < k; j += kSelectThreads) out[j] = j < n ? j : -1;
        return;
    }
    __shared__ SelectLds<kSelectThreads> sl;
    select_row<kSelectThreads>(scores + (int64_t)row * L, n, k, rw, lo.cap, out, sl);
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
                       hipStream_t stream, TopkState state, RowClear clear_after) {
    const Layout lo = make_layout(rows, L);
    const unsigned grid = (unsigned)((int64_t)rows * lo.nslice);
    if (state == TopkState::kNone) hipLaunchKernelGGL(topk_init_kernel, dim3(rows), dim3(kThreads), 0, stream, ws, lo);
    // finer LDS bins for long slices (measured: prefill 4096 x 128K rows, one slice per row)
    if (state != TopkState::kHistogram)
        hipLaunchKernelGGL(lo.slice >= kFineSlice ? topk_hist_kernel<13> : topk_hist_kernel<11>, dim3(grid),
                           dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws);
    hipLaunchKernelGGL(topk_filter_kernel, dim3(grid), dim3(kThreads), 0, stream, scores, q_pos, L, k, lo, ws,
                       state == TopkState::kHistogram ? 1 : 0);
    hipLaunchKernelGGL(topk_select_kernel, dim3(rows), dim3(kSelectThreads), 0, stream, scores, q_pos, L, k, lo, ws,
                       idx, clear_after);
    return hipGetLastError();
}

}  // namespace dsa
