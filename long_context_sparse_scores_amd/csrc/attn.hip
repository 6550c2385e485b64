// Sparse absorbed-MLA attention over the selected latent rows (gfx950).
//
// [TEARDOWN, 刀一 DSA] (clawlihai.cn GLM-5.2 1M architecture teardown): full
// attention runs over only the 2048 selected tokens.  [TEARDOWN, 刀三 MLA]:
// the cache keeps one compressed latent vector per token, shared by all 64
// heads (kv_lora_rank 512; with the 64-dim rope part a row holds 576 bf16).
// In absorbed form each head's query already lives in that latent space, so
//   z_j = sm_scale * <q_h, c_j>   (576 dims),   o_h = softmax(z) . c[:, 0:512].
//
// Work unit: one query (b,t) and a split of its index list; one workgroup per
// CU.  Selected rows are gathered 32 at a time (36 KiB tiles) straight from
// HBM into LDS with direct-to-LDS loads (no registers), four tile buffers
// deep so three tiles are in flight while one is computed.  The tile layout
// XOR-swizzles 16-byte chunks per row to spread operand reads over the LDS
// banks.  Per tile, with v_mfma_f32_16x16x32_bf16:
//   S^T (32 rows x 64 heads) = K_rows . Q^T   q in registers
//   O^T (512 dims x 64 heads) += V^T . P^T    V^T read with ds_read_b64_tr_b16,
//                                             P^T (bf16) through LDS
// The kernel splits this over eight waves in two roles, two waves per SIMD,
// so that one wave's Q.K^T and softmax run beside another's P.V (see below).
// Batches of fewer than 32 queries also split each query's 64 heads over two
// workgroups (head groups).
// Softmax is online in base 2 with a lazily moved reference maximum: the
// accumulators are rescaled only when a tile's maximum exceeds the reference
// by more than 32 (so P < 2^32 and the fp32 sums stay far from overflow);
// after the first tile this practically never happens.  Splits write
// normalised bf16 partial outputs plus their log2-sum-exp; a combine kernel,
// one block per (query, head), merges them in split order.  A query whose
// list fits one split is normalised and written directly.
//
// E4M3 latent rows ([CTXFR, "Entraînement par renforcement de l'agent
// intelligent"] names an FP8 KV cache) run through the same kernel
// (template parameter FP8): with 576-byte rows the LDS holds a ring of seven
// 18 KiB tiles, twice the rows in flight, and every operand is widened
// exactly to bf16 in registers as it is read, so the matrix cores compute as
// for bf16 rows.
#include <atomic>
#include <type_traits>

#include "common.h"

namespace dsa {
namespace {

constexpr int kHq = 64;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRows = 32;                         // gathered rows per tile
constexpr int kChunks = kDqk / 8;                 // 16-byte chunks per latent row (72)
constexpr int kTileChunks = kRows * kChunks;      // 2304 chunks = 36 KiB per tile
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLoads = 9;                         // direct-to-LDS loads per wave per tile: 8 row mains + 1 tail block
// Splits of a query's list (decode): row lists of up to 1024 entries, and 4
// bf16 tile buffers (3 tiles in flight) for splits of more than 4 tiles, else
// 3.  At the start every workgroup asks for its first tiles at once and that
// burst is bound by HBM, so a shorter burst lands tile 0 sooner, which pays
// when the split has few tiles to hide it behind (measured: 4-tile splits at
// B = 16, 21.4 -> 20.6 us per launch pair; 8-tile splits at B = 32, 31.4 us
// with 4 buffers against 31.9 with 3).  Whole lists (a query per workgroup,
// prefill sized batches): 3 buffers and up to 2048 entries; that path is bound
// by the matrix work, not by how many gathers are in flight.
template <bool DIRECT> struct Cfg {
    static constexpr int kMaxRows = DIRECT ? 2048 : 1024;
};
constexpr int kDirectStages = 3;
constexpr int kFewTiles = 4;  // splits of at most this many tiles take 3 buffers
constexpr int kMaxSplitRows = Cfg<false>::kMaxRows;
constexpr int kTargetBlocks = 256;                // one resident block per CU
// At most 16 splits per query: every split writes a 64 KiB partial that the
// combine reads back, and more, shorter splits cost more partials and combine
// rounds than they save (measured at 1M, B = 4: 64 splits of one tile 29 us per
// layer, 32 splits 19.8, 16 splits 18.4, 8 splits 20.6).
constexpr int kMaxQuerySplits = 16;
// A split launch whose bf16 row gathers come to at least this many bytes
// streams them past the caches (nontemporal loads).  Measured with four
// layers back to back: B = 32 at 128K (72 MiB of rows per launch), 27.9 ->
// 25.5 us per layer in the group step; B = 16 (36 MiB), 18.9 -> 20.5 us
// streamed, so smaller launches keep plain loads.
constexpr int64_t kStreamGatherBytes = 64ll << 20;
constexpr int kXcds = 8;                          // MI355X: 8 XCDs, block ids dealt round-robin
constexpr float kRescaleSlack = 32.0f;            // log2 units: P < 2^32, |O| < 2^46 in fp32

static_assert(kTileChunks % kThreads == 0, "tile load must split evenly");

// Tile layout in LDS (36 KiB for 32 rows): the first 64 chunks (1 KiB) of row r
// at byte r*1024 + 16*(c ^ (r & 15)) ("main"), the last 8 chunks at
// 32 KiB + r*128 + 16*((c - 64) ^ (r & 7)) ("tail").  The XORs spread the 16
// rows read by one MFMA operand over all LDS banks.  Value dims (the first 512)
// live in the main part only.
constexpr int kMainBytes = kRows * 1024;

// One 16-byte-per-lane direct-to-LDS load: lane l writes LDS bytes [lds + 16 l, lds + 16 l + 16).
// Issued from asm so that the compiler, which cannot tell which tile buffer the
// load fills, does not drain every in-flight load before each LDS read; the
// kernel orders these writes itself with wait_vmem() and lds_barrier().  The
// instruction has no register result and reads its address when issued.
// The statement sets m0 (the LDS destination) itself and lists it as clobbered.
// The compiler warns that it may not preserve a reserved register across asm;
// that is harmless here, because nothing else in these kernels keeps a value
// in m0: in their assembly every write of m0 is one of these statements.
// STREAM adds the nontemporal hint: the rows are read once, and they do not
// displace from the caches what the following kernels read back (the split
// partials, the next layer's inputs).
template <bool STREAM>
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_byte_addr) {
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(src), "s"(lds_byte_addr)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds_byte_addr)
                     : "memory", "m0");
}

// Same, with a wave-uniform 64-bit base and a per-lane 32-bit byte offset.
template <bool STREAM>
__device__ __forceinline__ void lds_dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_byte_addr) {
    if constexpr (STREAM)
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase),
                     "s"(lds_byte_addr)
                     : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_byte_addr)
                     : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}

// Gather of tile t (rows t*32 .. t*32+31 of this split) into LDS at `tile`.
// Wave w loads the main KiB of rows 8w .. 8w+7 (one load per row: lane l
// brings the row's 16-byte chunk l ^ (r & 15), which lands at tile byte
// 1024 r + 16 l) and the tails of the same 8 rows (one load).  Every lane
// holds its own source addresses, so making the plan is vector arithmetic on
// the row indices with no scalar dependency chain; only the LDS destinations
// are wave-uniform, and they do not depend on the row list.  rows_lds holds -1
// for every masked or missing entry (canonicalised when the list is loaded), so
// such rows read row 0; their scores are discarded and their value dims are
// cleared in LDS before P.V.
struct GatherPlan {
    const uint16_t* src[8];  // this lane's chunk of the main part of row 8w+i
    uint32_t lds[8];         // wave-uniform LDS byte addresses of the rows' main parts
    const uint16_t* tail;    // this lane's 16-byte tail chunk
    uint32_t lds_tail;
    bool active;             // wave-uniform: false when there is no tile left to gather
};

__device__ __forceinline__ GatherPlan plan_gather(const uint16_t* __restrict__ kvb, const int* __restrict__ rows_lds,
                                                  int t, const uint16_t* tile, int wave, int lane) {
    GatherPlan gp;
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(tile));
    const int r0 = 8 * wave;
    // the wave's 8 row indices in two 16-byte LDS reads (rows_lds is padded to whole tiles)
    const int4 ra = *reinterpret_cast<const int4*>(rows_lds + t * kRows + r0);
    const int4 rb = *reinterpret_cast<const int4*>(rows_lds + t * kRows + r0 + 4);
    const int rows8[8] = {ra.x, ra.y, ra.z, ra.w, rb.x, rb.y, rb.z, rb.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t rid = (uint32_t)max(rows8[i], 0);
        gp.src[i] = kvb + rid * kDqk + 8 * (lane ^ ((r0 + i) & 15));  // fits: L <= 2^22 rows
        gp.lds[i] = base + 1024u * (r0 + i);
    }
    {
        const int r = r0 + (lane >> 3);
        const uint32_t rid = (uint32_t)max(rows_lds[t * kRows + r], 0);
        const int c = 64 + ((lane & 7) ^ (r & 7));
        gp.tail = kvb + rid * kDqk + 8 * c;
        gp.lds_tail = base + kMainBytes + 1024u * wave;
    }
    gp.active = true;
    return gp;
}

// Load i of the plan: i < 8 the main part of row 8w+i, i == 8 the tails.
template <bool STREAM>
__device__ __forceinline__ void issue_gather(const GatherPlan& gp, int i) {
    if (!gp.active) return;
    lds_dma16<STREAM>(i < 8 ? gp.src[i] : gp.tail, i < 8 ? gp.lds[i] : gp.lds_tail);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even, one v_cvt_pk_bf16_f32), packed low-first.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

template <int N>
__device__ __forceinline__ void wait_vmem() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations
// only.  (__syncthreads() also waits for every outstanding global load,
// which would drain the gather pipeline.)  The asm memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Work split over the waves of a workgroup that takes HB head blocks (the
// score waves take the first two jobs, the value waves the third):
//   Q.K^T  score wave w < HB computes S^T for head block w (16 heads) over the
//          whole 576-dim contraction, the block's q in registers;
//   softmax  the same wave, into P^T (bf16) in LDS;
//   P.V    value wave w, value dims 128w .. 128w+127 of the HB head blocks,
//          with the P^T blocks read from LDS.
// Each active score wave reads the whole tile, so Q.K^T reads a tile from LDS
// HB times per workgroup and P.V once; in return no partial sums cross waves.
struct SoftmaxState {
    float m_ref;  // reference maximum (log2 units) of head 16w + c
    float lsum;   // this lane's share of the softmax denominator of head 16w + c
};

template <int HB> struct PvAcc {
    f32x4_t o[8][HB];  // O^T: value dims 128w + 16d + 4g + r of head 16hb + c of the workgroup's heads
};

// Per-lane LDS read addresses of one tile (bytes, relative to the tile), split
// into a lane base plus compile-time offsets.
//   S^T A operand, row rr = c (+16 per row block), chunk x = 4ks + g:
//     ks < 16: main, rr*1024 + 16*(16*(ks/4) + ((4*(ks%4) + g) ^ (rr & 15)))  -> qk[ks%4] + 256*(ks/4)
//     ks >= 16: tail, 32K + rr*128 + 16*((4*(ks-16) + g) ^ (rr & 7))         -> qt[ks-16]
//   V^T transpose read, row r = tr_row (+16), chunk 2db + q/2, byte 8*(q&1):
//     r*1024 + 16*(16*(db/8) + ((2*(db%8) + q/2) ^ (r & 15))) + 8*(q&1)       -> tr[db%8] + 256*(db/8)
struct TileAddr {
    int qk[4];
    int qt[2];
    int tr[8];
};

__device__ __forceinline__ TileAddr tile_addr(int lane) {
    const int c = lane & 15, g = lane >> 4;
    const int tr_row = 4 * g + ((lane & 15) >> 2);
    const int q = lane & 3;
    TileAddr a;
#pragma unroll
    for (int m = 0; m < 4; ++m) a.qk[m] = c * 1024 + 16 * ((4 * m + g) ^ (c & 15));
#pragma unroll
    for (int m = 0; m < 2; ++m) a.qt[m] = kMainBytes + c * 128 + 16 * ((4 * m + g) ^ (c & 7));
#pragma unroll
    for (int d = 0; d < 8; ++d) a.tr[d] = tr_row * 1024 + 16 * ((2 * d + (q >> 1)) ^ (tr_row & 15)) + 8 * (q & 1);
    return a;
}

// Online softmax of the S^T block of head block w for one tile (bit e of
// `valid`: value e of this lane is a visible row).  Updates the reference
// maximum and denominator share; when the reference moves, records the factor
// the P.V accumulators of these heads must be scaled by.  Returns P^T (k-slot
// 8g+e holds row e<4 ? 4g+e : 16+4g+e-4) in bf16.
__device__ __forceinline__ bf16x8_t softmax_tile(const f32x4_t (&s)[2], uint32_t valid, bool full, float scale_log2,
                                                 SoftmaxState& st, float& factor, bool& moved) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = s[e >> 2][e & 3] * scale_log2;
    if (!full) {  // wave-uniform: some row of the tile is masked (in place, so the paths share registers)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ((valid >> e) & 1u) ? x[e] : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    factor = 1.0f;
    moved = false;
    // The tile maximum over all lanes is only needed when the reference has to
    // move (the first tile with a visible row, or a jump beyond the slack).
    if (__ballot(mx > st.m_ref + kRescaleSlack)) {
        mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
        mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
        const float m_new = fmaxf(st.m_ref, mx);
        // While the reference is -inf nothing has been accumulated, so only a
        // finite old reference needs the accumulators rescaled.
        const bool scale = st.m_ref != -INFINITY && m_new != st.m_ref;
        if (__ballot(scale)) {
            factor = scale ? exp2f(st.m_ref - m_new) : 1.0f;
            st.lsum *= factor;
            moved = true;
        }
        st.m_ref = m_new;
    }
    const float mu = (st.m_ref == -INFINITY) ? 0.0f : st.m_ref;
    u32x4_t pw;
    const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        // v_exp_f32 directly: arguments are <= 32 here and results below 2^-126 may flush to 0
        const uint32_t h2 = pack_bf16x2(__builtin_amdgcn_exp2f(x[e] - mu), __builtin_amdgcn_exp2f(x[e + 1] - mu));
        // the denominator sums the bf16 values P uses: one v_dot2 with (1, 1) per pair
        st.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, h2), ones, st.lsum, false);
        pw[e / 2] = h2;
    }
    return __builtin_bit_cast(bf16x8_t, pw);
}

// Entry j of a split's row list as kept in LDS: the row, or -1 when it is
// missing (j >= nrows) or masked (outside [0, L)).
__device__ __forceinline__ int list_entry(const int32_t* sel, int j, int nrows, int L) {
    const int r = j < nrows ? sel[j] : -1;
    return (r >= 0 && r < L) ? r : -1;
}

// S^T of tile `tq` for one head block over the whole 576-dim contraction.
// qf[ks] holds the block's q for k-step ks; even and odd k-steps accumulate
// apart so that no MFMA waits on the one just issued, and the two halves are
// summed at the end.
__device__ __forceinline__ void qk_full(const uint16_t* tq, const TileAddr& ad, const bf16x8_t (&qf)[kDqk / 32],
                                        f32x4_t (&s)[2]) {
    f32x4_t acc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[rb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) {
        const int off = ks < 16 ? ad.qk[ks & 3] + 256 * (ks >> 2) : ad.qt[ks - 16];
        const int rb1 = ks < 16 ? 16 * 1024 : 16 * 128;  // next row block: tail rows are 128 B
        const char* p = reinterpret_cast<const char*>(tq) + off;
        const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(p);
        const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(p + rb1);
        acc[0][ks & 1] = mfma16x16x32(a0, qf[ks], acc[0][ks & 1]);
        acc[1][ks & 1] = mfma16x16x32(a1, qf[ks], acc[1][ks & 1]);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) s[rb] = acc[rb][0] + acc[rb][1];
}

// Output rows staged in LDS by the epilogue: 64 rows of 512 bf16, padded to
// 1040 bytes so that the 8-byte staging writes hit every bank once (65 KiB).
constexpr int kStageRow = 2 * kDv + 16;

// ------------------------------------------------------------------ P.V helpers of the bf16 tiles
template <int HB>
__device__ __forceinline__ void load_p(const bf16x8_t* __restrict__ pl, int lane, bf16x8_t (&pbv)[HB]) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) pbv[hb] = pl[hb * kWave + lane];
}

// P.V of tile tv for value dims 128 vw .. +127 of the workgroup's HB head blocks.
template <int HB>
__device__ __forceinline__ void pv_tile(const uint16_t* tv, const TileAddr& ad, const bf16x8_t (&pbv)[HB], int vw,
                                        PvAcc<HB>& acc) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {
        const char* p = reinterpret_cast<const char*>(tv) + ad.tr[d] + 256 * vw;
        const bf16x4_t lo = lds_read_tr16(p);
        const bf16x4_t hi = lds_read_tr16(p + 16 * 1024);
        const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc.o[d][hb] = mfma16x16x32(a, pbv[hb], acc.o[d][hb]);
    }
}

// ------------------------------------------------------------------ E4M3 latent rows
// A 32-row tile of 576-byte E4M3 rows is 18 KiB, so the LDS holds a ring of
// seven: six tiles in flight while one is read, twice the rows in flight of
// the bf16 tiles.  The work split, softmax and combine are the same; only the
// gathers and the operand reads differ, each operand widened exactly to bf16
// in registers (v_cvt_scalef32_pk_bf16_fp8 with a scale of 1, two codes per
// instruction):
//   Q.K^T  A operand, 8 dims of a row: one ds_read_b64;
//   P.V    A operand, 8 rows of one dim: one ds_read_b64_tr_b8 (in each
//          16-lane group, lane 8q + r receives byte r of the 8-byte chunks
//          addressed by lanes 2j + q, as value j = 0..7), with the rows in the
//          order of the P^T k-slots.
// Chunk s (16 bytes) of row r sits at byte 16 * (36r + (s ^ f(r))),
// f(r) = ((r >> 2) + 2(r >> 4)) & 3: both reads touch every LDS bank once per
// 32-lane phase (checked by enumeration).  A tile's rescale record lives in a
// small array beside the ring.
constexpr int kRow8 = kDqk;                       // bytes per E4M3 row
constexpr int kChunks8 = kRow8 / 16;              // 36
constexpr int kTile8Bytes = kRows * kRow8;        // 18 KiB
constexpr int kStages8 = 7;
constexpr int kLoads8Max = 5;                     // 18 wave loads of 1 KiB per tile: 5, 5, 4, 4 over the waves

__device__ __forceinline__ int swz8(int r) { return ((r >> 2) + 2 * (r >> 4)) & 3; }

// Gather of E4M3 tile t: load n (wave n % 4) fills slots 64n .. 64n+63 of the
// tile (1 KiB); the lane writing slot P fetches the chunk stored there.
struct GatherPlan8 {
    const uint8_t* base;       // wave-uniform: the sequence's first row
    uint32_t off[kLoads8Max];  // this lane's byte offsets from base
    uint32_t lds[kLoads8Max];  // wave-uniform LDS byte address of each load
    int nload;                 // wave-uniform: 5 or 4
    bool active;
};

__device__ __forceinline__ GatherPlan8 plan_gather8(const uint8_t* __restrict__ kvb, const int* __restrict__ rows_lds,
                                                    int t, const uint8_t* tile, int wave, int lane) {
    GatherPlan8 gp;
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_address(tile));
    gp.base = kvb;
    gp.nload = wave < 2 ? 5 : 4;
#pragma unroll
    for (int i = 0; i < kLoads8Max; ++i) {
        const int n = wave + 4 * i;                 // < 18 for the loads this wave issues
        const int slot = 64 * n + lane;
        const int r = min(slot / kChunks8, kRows - 1);
        // rows_lds holds -1 for masked or missing rows: they read row 0 (scores discarded, values cleared)
        const uint32_t rid = (uint32_t)max(rows_lds[t * kRows + r], 0);
        const int s = (slot - kChunks8 * r) ^ swz8(r);
        gp.off[i] = slot < kRows * kChunks8 ? rid * kRow8 + 16u * (uint32_t)s : 0u;  // L <= 2^22 rows
        gp.lds[i] = __builtin_amdgcn_readfirstlane(base + 1024u * n);
    }
    gp.active = true;
    return gp;
}

template <bool STREAM>
__device__ __forceinline__ void issue_gather(const GatherPlan8& gp, int i) {
    if (!gp.active || i >= gp.nload) return;
    lds_dma16_sbase<STREAM>(gp.base, gp.off[i], gp.lds[i]);
}

// Wait until at most `tiles` (0..5) E4M3 tile gathers of this wave, of nload
// loads each (5 or 4; both wave-uniform), are still in flight.
__device__ __forceinline__ void wait_tiles8(int tiles, int nload) {
    if (nload == 5) {
        if (tiles <= 0) wait_vmem<0>();
        else if (tiles == 1) wait_vmem<5>();
        else if (tiles == 2) wait_vmem<10>();
        else if (tiles == 3) wait_vmem<15>();
        else if (tiles == 4) wait_vmem<20>();
        else wait_vmem<25>();
    } else {
        if (tiles <= 0) wait_vmem<0>();
        else if (tiles == 1) wait_vmem<4>();
        else if (tiles == 2) wait_vmem<8>();
        else if (tiles == 3) wait_vmem<12>();
        else if (tiles == 4) wait_vmem<16>();
        else wait_vmem<20>();
    }
}

typedef int i32x2_t __attribute__((ext_vector_type(2)));

// 8 E4M3 codes (low byte first) -> 8 bf16, exactly: one v_cvt_scalef32_pk_bf16_fp8
// per pair with a scale of 1 (every E4M3 value, subnormals included, is a
// bf16 value), the lower code into the lower half.
__device__ __forceinline__ bf16x8_t e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3), __builtin_shufflevector(c, d, 0, 1, 2, 3),
                                   0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-lane parts of the operand addresses (bytes within a tile).
struct TileAddr8 {
    int qk;    // 576c + 8(g & 1): rows c and c + 16, half g & 1 of their chunks
    int fq0;   // swz8(c), swz8(c + 16)
    int fq1;
    int pv;    // 576 r + 8 (m & 1) for the P.V row r of this lane
    int fpv;   // swz8(r)
};

__device__ __forceinline__ TileAddr8 tile_addr8(int lane) {
    const int c = lane & 15, g = lane >> 4;
    TileAddr8 a;
    a.qk = kRow8 * c + 8 * (g & 1);
    a.fq0 = swz8(c);
    a.fq1 = swz8(c + 16);
    // lane m of group g addresses k-slot j = m >> 1 of the P^T ordering:
    // row 4g + j for j < 4, row 16 + 4g + j - 4 otherwise; half m & 1
    const int m = lane & 15, j = m >> 1;
    const int r = j < 4 ? 4 * g + j : 16 + 4 * g + j - 4;
    a.pv = kRow8 * r + 8 * (m & 1);
    a.fpv = swz8(r);
    return a;
}

struct RescaleRecord {
    float fac[4 * 16];  // per head block, per head
    uint32_t flag[4];   // block hb moved its reference
};

template <int HB>
__device__ __forceinline__ void apply_rescale(const RescaleRecord& rs, int c, PvAcc<HB>& acc) {
    const u32x4_t fl = *reinterpret_cast<const u32x4_t*>(rs.flag);
    const uint32_t any = __builtin_amdgcn_readfirstlane(fl[0] | (HB > 1 ? fl[1] : 0u) | (HB > 2 ? fl[2] | fl[3] : 0u));
    if (any) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            if (__builtin_amdgcn_readfirstlane(fl[hb])) {
                const float f = rs.fac[16 * hb + c];
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    acc.o[d][hb] *= f;
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
}

// S^T of E4M3 tile `tq` for one head block over the whole contraction (the
// rows widened exactly to bf16 as they are read), in the same order of MFMAs
// and sums as qk_full, so both caches give bit-identical scores for the same
// values.
__device__ __forceinline__ void qk_full8(const uint8_t* tq, const TileAddr8& ad, const bf16x8_t (&qf)[kDqk / 32], int g,
                                         f32x4_t (&s)[2]) {
    f32x4_t acc[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int h = 0; h < 2; ++h) acc[rb][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) {
        const int ch = 2 * ks + (g >> 1);  // chunk of dims 32ks + 8g .. +7
        const uint2 r0 = *reinterpret_cast<const uint2*>(tq + ad.qk + 16 * (ch ^ ad.fq0));
        const uint2 r1 = *reinterpret_cast<const uint2*>(tq + ad.qk + 16 * kRow8 + 16 * (ch ^ ad.fq1));
        acc[0][ks & 1] = mfma16x16x32(e4m3x8_to_bf16x8(r0.x, r0.y), qf[ks], acc[0][ks & 1]);
        acc[1][ks & 1] = mfma16x16x32(e4m3x8_to_bf16x8(r1.x, r1.y), qf[ks], acc[1][ks & 1]);
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) s[rb] = acc[rb][0] + acc[rb][1];
}

// P.V of E4M3 tile tv for value dims 128 vw .. +127 of the workgroup's HB head blocks.
template <int HB>
__device__ __forceinline__ void pv_tile8(const uint8_t* tv, const TileAddr8& ad, const bf16x8_t (&pbv)[HB], int vw,
                                         PvAcc<HB>& acc) {
#pragma unroll
    for (int d = 0; d < 8; ++d) {  // value dims 128 vw + 16 d .. +15: chunk 8 vw + d
        const i32x2_t raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(tv + ad.pv + 16 * ((8 * vw + d) ^ ad.fpv)));
        const bf16x8_t a = e4m3x8_to_bf16x8((uint32_t)raw[0], (uint32_t)raw[1]);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc.o[d][hb] = mfma16x16x32(a, pbv[hb], acc.o[d][hb]);
    }
}

// The gather plan of tile t into LDS buffer `tile` for value wave vw (bf16 or E4M3 rows).
template <bool FP8>
__device__ __forceinline__ auto plan_tile(const void* kvb, const int* rows_lds, int t, uint8_t* tile, int vw,
                                          int lane) {
    if constexpr (FP8) return plan_gather8(reinterpret_cast<const uint8_t*>(kvb), rows_lds, t, tile, vw, lane);
    else return plan_gather(reinterpret_cast<const uint16_t*>(kvb), rows_lds, t, reinterpret_cast<uint16_t*>(tile),
                            vw, lane);
}

// Wait until at most `tiles_left` of this value wave's tile gathers are in flight.
template <bool FP8>
__device__ __forceinline__ void wait_gathers(int tiles_left, int nload) {
    if constexpr (FP8) {
        wait_tiles8(tiles_left, nload);
    } else {
        (void)nload;
        if (tiles_left >= 2) wait_vmem<2 * kLoads>();
        else if (tiles_left == 1) wait_vmem<kLoads>();
        else wait_vmem<0>();
    }
}

// ------------------------------------------------------------------ merging the splits of a query
// With lse_s the log2-sum-exp of split s and O_s its normalised partial,
//   out = sum_s 2^(lse_s - M) O_s / sum_s 2^(lse_s - M),   M = max_s lse_s,
// the numerator summed in split order.  One wave per (query, head), 8 value
// dims per lane: lane s holds split s's log2-sum-exp, the maximum and the
// denominator come from wave reductions, the weights reach the accumulation
// through readlane, and the loads of all NB >= nsplit partials go out first
// (NB = 8 when there are at most 8 splits, else 16).
constexpr int kCombineNB = 8;
static_assert(kWave * 8 == kDv, "8 value dims per lane");

template <int NB>
__device__ __forceinline__ void combine_head(const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
                                             int bt, int head, int nsplit, uint16_t* __restrict__ out,
                                             float* __restrict__ lse, int lane) {
    static_assert(kMaxQuerySplits <= 16 && kMaxQuerySplits <= kWave, "one load round, one lane per split");
    // split s of this (query, head): partial at po + s * kHq * kDv bf16, log2-sum-exp at pl + s * kHq
    const __amdgpu_buffer_rsrc_t po = wt_rsrc(part_o + ((int64_t)bt * nsplit * kHq + head) * kDv);
    const __amdgpu_buffer_rsrc_t pl = wt_rsrc(part_lse + (int64_t)bt * nsplit * kHq + head);
    // the split weights first: their reductions run while the partials are in flight
    const float ls =
        lane < nsplit ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(pl, (int)(4u * (uint32_t)(lane * kHq)), 0, 0))
                      : -INFINITY;
    u32x4_t v[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int sp = min(u, nsplit - 1);  // past the end: a valid split, weight 0 below
        v[u] = __builtin_bit_cast(u32x4_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(po, (int)(2u * (uint32_t)(sp * kHq * kDv + 8 * lane)), 0, 0));
    }
    float M = ls;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
    const float a = (ls == -INFINITY) ? 0.0f : exp2f(ls - M);  // M == -inf only when every split is empty
    float den = a;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) den += __shfl_xor(den, off, kWave);
    const uint32_t a_bits = __float_as_uint(a);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const float w = u < nsplit ? __uint_as_float(__builtin_amdgcn_readlane(a_bits, u)) : 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += w * __uint_as_float(v[u][e] << 16);
            acc[2 * e + 1] += w * __uint_as_float(v[u][e] & 0xFFFF0000u);
        }
    }
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    store_wt16(wt_rsrc(out + ((int64_t)bt * kHq + head) * kDv), 16u * lane, o);
    if (lse && lane == 0)
        store_wt4(wt_rsrc(lse + (int64_t)bt * kHq), 4u * head,
                  den > 0.0f ? (M + log2f(den)) * 0.69314718055994531f : -INFINITY);
}

// ------------------------------------------------------------------ the attention kernel: two roles per SIMD
// Eight waves, two per SIMD.  A workgroup takes one query, a split of its
// index list and HB of its four 16-head blocks (heads 16 HB hg .. +16 HB - 1 for
// head group hg).  Waves 0-3 ("score waves"): wave w < HB computes S^T of head
// block w over the whole 576-dim contraction, q in registers, and runs its
// softmax; waves 4-7 ("value waves") issue the gathers and do P.V for value
// dims 128(w-4) .. +127 of the HB head blocks.  One workgroup barrier per tile
// step; between two of them
//   score waves: Q.K^T and softmax of tile t+1 (P^T and rescale record to LDS
//                at parity (t+1) & 1);
//   value waves: the gathers of tile t+kStages-1 (planned one iteration
//                earlier), tile t's rescale record applied and its P^T blocks
//                loaded, the next gather plan beside P.V of tile t, then the
//                wait for their loads of tile t+1.
// So on every SIMD one wave's Q.K^T and softmax run beside the other's P.V.
// Each score wave reads the whole tile from LDS; no partial sums cross waves.
// Head groups (HB < 4) let small batches spread a query over more
// workgroups without more split partials: the groups of a query gather the
// same rows, on one XCD, so all but the first read of a row come from its L2.
// The two roles run separate loops with the same sequence of barriers, so the
// registers of one (q for the score waves, the accumulators for the value
// waves) are not held by the other.
// FP8: the latent rows are E4M3 codes in a ring of seven 18 KiB tiles;
// otherwise bf16 tiles (the bf16 decode configuration uses 157 of 160 KiB).
template <bool DIRECT, bool FP8, int STAGES, bool STREAM = false, int HB = 4>
__global__ __launch_bounds__(2 * kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv_any, int64_t kv_bstride,
    const int32_t* __restrict__ idx, int rows, int T, int L, int k, int rows_per_split, int nsplit, float scale_log2,
    uint16_t* __restrict__ part_o, float* __restrict__ part_lse, uint16_t* __restrict__ out, float* __restrict__ lse) {
    static_assert(HB == 1 || HB == 2 || HB == 4, "head blocks per workgroup");
    constexpr int kGroups = 4 / HB;  // head groups per query
    const int nparts = nsplit * kGroups;
    const int grp = blockIdx.x / (kXcds * nparts);
    const int rem = blockIdx.x % (kXcds * nparts);
    const int part = rem / kXcds;
    const int split = part / kGroups;
    const int h0 = 16 * HB * (part % kGroups);  // first head of this workgroup
    const int bt = grp * kXcds + rem % kXcds;
    if (bt >= rows) return;
    const int b = bt / T;
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool score = wave < kWaves;
    const int c = lane & 15;
    const int g = lane >> 4;
    const int j0 = split * rows_per_split;
    const int nrows = min(k, j0 + rows_per_split) - j0;
    const int ntiles = (nrows + kRows - 1) / kRows;

    constexpr int kStages = FP8 ? kStages8 : STAGES;  // tile buffers
    constexpr int kTileBytes = FP8 ? kTile8Bytes : kTileChunks * 16;
    using TileT = typename std::conditional<FP8, uint8_t, uint16_t>::type;
    __shared__ __attribute__((aligned(16))) TileT tiles[kStages * kTileBytes / sizeof(TileT)];
    static_assert(kHq * kStageRow <= (int)sizeof(tiles), "the output staging fits in the tile buffers");
    // P^T and the rescale record of tile t at parity t & 1: the score waves
    // write tile t+1's while the value waves read tile t's.
    __shared__ __attribute__((aligned(16))) bf16x8_t pl[2 * HB * kWave];  // P^T of the HB head blocks
    __shared__ __attribute__((aligned(16))) int rows_lds[Cfg<DIRECT>::kMaxRows];
    __shared__ __attribute__((aligned(16))) RescaleRecord records[2];
    __shared__ __attribute__((aligned(16))) float stats[2 * kHq];  // epilogue: [0, 64) sums, [64, 128) maxima
    auto buf = [&](int t) __attribute__((always_inline)) {
        return reinterpret_cast<uint8_t*>(tiles) + (t % kStages) * kTileBytes;
    };
    auto buf16 = [&](int t) __attribute__((always_inline)) {
        return reinterpret_cast<const uint16_t*>(tiles) + (t % kStages) * (kTileBytes / 2);
    };
    const TileAddr ad = tile_addr(lane);     // bf16 operand addresses
    const TileAddr8 ad8 = tile_addr8(lane);  // E4M3 operand addresses
    char* st8 = reinterpret_cast<char*>(tiles);  // epilogue: output rows staged, kStageRow bytes apart

    const int32_t* sel = idx + (int64_t)bt * k + j0;
    if (score) {
        // ---------------- score waves: wave sw < HB, head block sw of the group
        const int sw = wave;
        const bool active = sw < HB;  // wave-uniform
        // The row list is read before q: loads return in order, and the list
        // is what the gathers wait for, while q is first needed by tile 0's Q.K^T.
        constexpr int kListPer = Cfg<DIRECT>::kMaxRows / (2 * kThreads);
        int le[kListPer];
#pragma unroll
        for (int u = 0; u < kListPer; ++u) {
            const int j = threadIdx.x + 2 * kThreads * u;
            le[u] = j < ntiles * kRows ? list_entry(sel, j, nrows, L) : -1;
        }
        bf16x8_t qf[kDqk / 32];
        if (active) {
            const uint16_t* qh = q + ((int64_t)bt * kHq + h0 + 16 * sw + c) * kDqk + 8 * g;
#pragma unroll
            for (int ks = 0; ks < kDqk / 32; ++ks) qf[ks] = *reinterpret_cast<const bf16x8_t*>(qh + 32 * ks);
        }
#pragma unroll
        for (int u = 0; u < kListPer; ++u) {
            const int j = threadIdx.x + 2 * kThreads * u;
            if (j < ntiles * kRows) rows_lds[j] = le[u];
        }
        __syncthreads();  // rows_lds ready
        SoftmaxState st;
        st.m_ref = -INFINITY;
        st.lsum = 0.0f;
        // Q.K^T of tile t and the softmax; P^T and the rescale record to LDS
        auto scores_of = [&](int t) __attribute__((always_inline)) {
            if (!active) return;
            // the tile's visible rows: one LDS read and a ballot give a wave-uniform mask
            const uint32_t tmask = (uint32_t)__ballot(rows_lds[t * kRows + (lane & 31)] >= 0);
            f32x4_t s[2];
            if constexpr (FP8) qk_full8(buf(t), ad8, qf, g, s);
            else qk_full(buf16(t), ad, qf, s);
            // value e of this lane is row e < 4 ? 4g + e : 16 + 4g + e - 4
            const uint32_t valid = ((tmask >> (4 * g)) & 0xFu) | (((tmask >> (16 + 4 * g)) & 0xFu) << 4);
            float factor;
            bool moved;
            const bf16x8_t pb = softmax_tile(s, valid, tmask == 0xFFFFFFFFu, scale_log2, st, factor, moved);
            pl[((t & 1) * HB + sw) * kWave + lane] = pb;
            if (g == 0) records[t & 1].fac[16 * sw + c] = factor;
            if (lane == 0) records[t & 1].flag[sw] = moved ? 1u : 0u;
        };
        lds_barrier();  // tile 0 in LDS
        scores_of(0);
        for (int t = 0; t + 1 < ntiles; ++t) {
            lds_barrier();  // tile t+1 in LDS; P^T of tile t-1 read by the value waves
            scores_of(t + 1);
        }
        lds_barrier();  // P^T and rescale record of the last tile visible
        // epilogue: denominators and maxima of head block sw
        float lsum = st.lsum;
        lsum += __shfl_xor(lsum, 16, kWave);
        lsum += __shfl_xor(lsum, 32, kWave);
        const int head = h0 + 16 * sw + c;
        if (active && g == 0) {
            stats[16 * sw + c] = lsum;
            stats[64 + 16 * sw + c] = st.m_ref;
            // the log-sum-exp goes out now, beside the value waves' staging
            if (DIRECT) {
                if (lse)
                    store_wt4(wt_rsrc(lse + (int64_t)bt * kHq), 4u * head,
                              lsum > 0.0f ? (st.m_ref + log2f(lsum)) * 0.69314718055994531f : -INFINITY);
            } else {
                store_wt4(wt_rsrc(part_lse + ((int64_t)bt * nsplit + split) * kHq), 4u * head,
                          lsum > 0.0f ? st.m_ref + log2f(lsum) : -INFINITY);
            }
        }
        lds_barrier();  // stats visible
        lds_barrier();  // output rows staged
    } else {
        // ---------------- value waves
        const int vw = wave - kWaves;
        // the sequence's rows (bf16 strides count elements, E4M3 strides bytes)
        const void* kvb = FP8 ? (const void*)(reinterpret_cast<const uint8_t*>(kv_any) + b * kv_bstride)
                              : (const void*)(reinterpret_cast<const uint16_t*>(kv_any) + b * kv_bstride);
        const int nload = FP8 ? (vw < 2 ? 5 : 4) : kLoads;  // loads per tile of this wave
        constexpr int kMaxLoads = FP8 ? kLoads8Max : kLoads;
        static_assert(FP8 || (STAGES >= 3 && STAGES <= 4), "bf16 wait counts cover one or two later tiles in flight");
        for (int j = threadIdx.x; j < ntiles * kRows; j += 2 * kThreads) rows_lds[j] = list_entry(sel, j, nrows, L);
        __syncthreads();  // rows_lds ready
        // Masked or missing entries gather row 0, and their scores are discarded;
        // their value rows are cleared before P.V (P = 0 would not hide an Inf or
        // NaN there).  Wave vw clears the rows r = vw (mod 4) of tile t.
        auto clear_masked = [&](int t) __attribute__((always_inline)) {
            uint32_t m = ~(uint32_t)__ballot(rows_lds[t * kRows + (lane & 31)] >= 0) & (0x11111111u << vw);
            while (m) {
                const int r = __builtin_ctz(m);
                m &= m - 1;
                if constexpr (FP8) {  // value bytes 0..511: chunk positions 36r .. 36r+31
                    if (lane < 32) *reinterpret_cast<u32x4_t*>(buf(t) + kRow8 * r + 16 * lane) = u32x4_t{0u, 0u, 0u, 0u};
                } else {              // the 1 KiB main part holds the 512 value dims
                    *reinterpret_cast<u32x4_t*>(buf(t) + 1024 * r + 16 * lane) = u32x4_t{0u, 0u, 0u, 0u};
                }
            }
        };
        for (int t = 0; t < kStages - 1 && t < ntiles; ++t) {
            const auto gp = plan_tile<FP8>(kvb, rows_lds, t, buf(t), vw, lane);
#pragma unroll
            for (int i = 0; i < kMaxLoads; ++i) issue_gather<STREAM>(gp, i);
        }
        PvAcc<HB> acc;
#pragma unroll
        for (int d = 0; d < 8; ++d)
#pragma unroll
            for (int hb = 0; hb < HB; ++hb) acc.o[d][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        wait_gathers<FP8>(min(ntiles - 1, kStages - 2), nload);  // tile 0 landed
        // The plan of each in-loop gather (addresses from rows_lds) is made one
        // iteration ahead, beside the P.V work, so the loop head only issues the loads.
        auto next = plan_tile<FP8>(kvb, rows_lds, min(kStages - 1, ntiles - 1), buf(kStages - 1), vw, lane);
        next.active = kStages - 1 < ntiles;
        lds_barrier();  // tile 0 in LDS
        clear_masked(0);  // beside the score waves' Q.K^T, whose masked scores are discarded
        bf16x8_t pbv[HB];
        for (int t = 0; t + 1 < ntiles; ++t) {
            // this thread's loads of tile t+1 are done once only those of later tiles are outstanding
            wait_gathers<FP8>(min(ntiles - 1, t + kStages - 2) - (t + 1), nload);
            lds_barrier();  // tile t+1 in LDS; P^T and rescale record of tile t visible; buffer t-1 free
#pragma unroll
            for (int i = 0; i < kMaxLoads; ++i) issue_gather<STREAM>(next, i);  // tile t + kStages - 1
            apply_rescale<HB>(records[t & 1], c, acc);
            load_p<HB>(pl + (t & 1) * HB * kWave, lane, pbv);
            // tile t + kStages goes to this tile's buffer, next iteration, after this P.V and a barrier
            auto nx = plan_tile<FP8>(kvb, rows_lds, min(t + kStages, ntiles - 1), buf(t), vw, lane);
            nx.active = t + kStages < ntiles;
            if constexpr (FP8) pv_tile8<HB>(buf(t), ad8, pbv, vw, acc);
            else pv_tile<HB>(buf16(t), ad, pbv, vw, acc);
            // before tile t+1's P.V, after the next barrier; beside its Q.K^T, whose
            // masked scores are discarded
            clear_masked(t + 1);
            next = nx;
        }
        lds_barrier();  // P^T and rescale record of the last tile visible
        apply_rescale<HB>(records[(ntiles - 1) & 1], c, acc);
        load_p<HB>(pl + ((ntiles - 1) & 1) * HB * kWave, lane, pbv);
        if constexpr (FP8) pv_tile8<HB>(buf(ntiles - 1), ad8, pbv, vw, acc);
        else pv_tile<HB>(buf16(ntiles - 1), ad, pbv, vw, acc);
        lds_barrier();  // stats visible; every value wave is done reading the tiles
        float inv[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
            const float ls = stats[16 * hb + c];
            inv[hb] = ls > 0.0f ? 1.0f / ls : 0.0f;
        }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb)
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const f32x4_t& o = acc.o[d][hb];
                *reinterpret_cast<uint2*>(st8 + (16 * hb + c) * kStageRow + 2 * (128 * vw + 16 * d + 4 * g)) =
                    make_uint2(pack_bf16x2(o[0] * inv[hb], o[1] * inv[hb]), pack_bf16x2(o[2] * inv[hb], o[3] * inv[hb]));
            }
        lds_barrier();  // output rows staged
    }
    // every wave stores 2 HB of the 16 HB head rows, one 16-byte store per lane per row
    const __amdgpu_buffer_rsrc_t dst = wt_rsrc(DIRECT ? out + ((int64_t)bt * kHq + h0) * kDv
                                                      : part_o + (((int64_t)bt * nsplit + split) * kHq + h0) * kDv);
#pragma unroll
    for (int i = 0; i < 2 * HB; ++i) {
        const int h = 2 * HB * wave + i;
        store_wt16(dst, 2u * (h * kDv + 8 * lane), *reinterpret_cast<const u32x4_t*>(st8 + h * kStageRow + 16 * lane));
    }
}

// The split partials merged in a launch of their own: one wave per (query,
// head), blocks numbered like the split kernel.  (Merging inside the split
// launch instead, each split merging a group of heads once all splits of its
// query had written their partials, measured 0.5 us per layer slower at
// decode 128K x 32.)
constexpr int kCombineThreads = kWave;

template <int NB>
__global__ __launch_bounds__(kCombineThreads) void attn_combine_kernel(const uint16_t* __restrict__ part_o,
                                                                       const float* __restrict__ part_lse, int rows,
                                                                       int nsplit, uint16_t* __restrict__ out,
                                                                       float* __restrict__ lse) {
    const int grp = blockIdx.x / (kXcds * kHq);
    const int rem = blockIdx.x % (kXcds * kHq);
    const int head = rem / kXcds;
    const int bt = grp * kXcds + rem % kXcds;
    if (bt >= rows) return;
    combine_head<NB>(part_o, part_lse, bt, head, nsplit, out, lse, lane_id());
}

unsigned xcd_grid(int rows, int per_row) {
    return (unsigned)((int64_t)((rows + kXcds - 1) / kXcds) * kXcds * per_row);
}

struct SplitPlan {
    int nsplit, rows_per_split;
    int hgroups;  // head groups per query: 1, 2 or 4 workgroups share a split's rows
};

// Splits of about `ns` per query (clamped so that every split's row list fits
// the split kernel's LDS and holds at least one tile).
SplitPlan plan_splits(int rows, int k, int ns) {
    (void)rows;
    const int tiles = (k + kRows - 1) / kRows;
    if (ns > kMaxQuerySplits) ns = kMaxQuerySplits;
    if (ns > 1) {  // split lists: each split's row list fits the split kernel's LDS
        const int min_ns = (tiles * kRows + kMaxSplitRows - 1) / kMaxSplitRows;
        if (ns < min_ns) ns = min_ns;
    }
    if (ns > tiles) ns = tiles;
    if (ns < 1) ns = 1;
    const int tiles_per = (tiles + ns - 1) / ns;
    const int rps = tiles_per * kRows;
    return SplitPlan{(k + rps - 1) / rps, rps, 1};
}

// Batches of fewer than kGroupRows queries split each query's heads over two
// workgroups (head groups), and take splits for about kTargetBlocks
// workgroups in all.  Measured against whole-query workgroups (attention
// launch pair per layer or draft step):
//   B = 16, 128K: 8 splits x 2 groups against 16 splits, 19.4 -> 17.8 us;
//   B = 4, 1M: 16 splits x 2 groups against 16 splits, 17.9 -> 16.3 us; with
//   4 groups (256 workgroups) 20.7 us, with 8 splits x 2 groups 18.1 us.
// At B = 32 (8 splits) 4 splits x 2 groups measured the same as 8 splits, so
// full batches keep whole-query workgroups.
constexpr int kGroupRows = 32;

// The partials' layout: splits (and head groups) for about kTargetBlocks
// workgroups.
SplitPlan plan(int rows, int k) {
    const int hg = rows < kGroupRows ? 2 : 1;
    SplitPlan p = plan_splits(rows, k, (kTargetBlocks + rows * hg - 1) / (rows * hg));
    p.hgroups = hg;
    return p;
}

// Workspace: [partials bf16][log2-sum-exps fp32], 256-byte aligned parts.
struct AttnWs {
    uint16_t* part_o;
    float* part_lse;
};

size_t part_o_bytes(int rows, int k) {
    return align_up((size_t)rows * plan(rows, k).nsplit * kHq * kDv * sizeof(uint16_t), 256);
}
size_t part_lse_bytes(int rows, int k) {
    return align_up((size_t)rows * plan(rows, k).nsplit * kHq * sizeof(float), 256);
}

AttnWs attn_ws(void* ws, int rows, int k) {
    char* b = reinterpret_cast<char*>(ws);
    return AttnWs{reinterpret_cast<uint16_t*>(b), reinterpret_cast<float*>(b + part_o_bytes(rows, k))};
}

template <bool DIRECT, bool FP8, int STAGES, bool STREAM>
using AttnKernel = decltype(&sparse_mla_kernel<DIRECT, FP8, STAGES, STREAM, 4>);

// The kernel instance for `hgroups` (1 or 2) head groups of 4 / hgroups head blocks.
template <bool DIRECT, bool FP8, int STAGES, bool STREAM = false>
AttnKernel<DIRECT, FP8, STAGES, STREAM> attn_kernel(int hgroups) {
    return hgroups == 2 ? sparse_mla_kernel<DIRECT, FP8, STAGES, STREAM, 2>
                        : sparse_mla_kernel<DIRECT, FP8, STAGES, STREAM, 4>;
}

template <bool FP8, typename KV>
hipError_t launch_attn_impl(const uint16_t* q, const KV* kv, int64_t kv_bstride, const int32_t* idx, int B, int T,
                            int L, int k, float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
    const int rows = B * T;
    const float scale_log2 = sm_scale * 1.4426950408889634f;
    const SplitPlan p = plan(rows, k);
    if (p.nsplit == 1) {
        const auto direct_kernel = attn_kernel<true, FP8, FP8 ? kStages8 : kDirectStages>(p.hgroups);
        hipLaunchKernelGGL(direct_kernel, dim3(xcd_grid(rows, p.hgroups)), dim3(2 * kThreads), 0, stream, q, kv, kv_bstride, idx, rows,
                           T, L, k, p.rows_per_split, 1, scale_log2, nullptr, nullptr, out, lse);
        return hipGetLastError();
    }
    const AttnWs w = attn_ws(ws, rows, k);
    AttnKernel<false, FP8, 3, false> split_kernel;
    if constexpr (FP8) split_kernel = attn_kernel<false, true, kStages8>(p.hgroups);
    else if (p.rows_per_split <= kFewTiles * kRows) split_kernel = attn_kernel<false, false, 3>(p.hgroups);
    else if ((int64_t)rows * k * kDqk * 2 >= kStreamGatherBytes) split_kernel = attn_kernel<false, false, 4, true>(p.hgroups);
    else split_kernel = attn_kernel<false, false, 4>(p.hgroups);
    hipLaunchKernelGGL(split_kernel, dim3(xcd_grid(rows, p.nsplit * p.hgroups)), dim3(2 * kThreads), 0, stream, q, kv,
                       kv_bstride, idx, rows, T, L, k, p.rows_per_split, p.nsplit, scale_log2, w.part_o, w.part_lse,
                       out, lse);
    hipLaunchKernelGGL(p.nsplit <= kCombineNB ? attn_combine_kernel<kCombineNB> : attn_combine_kernel<kMaxQuerySplits>,
                       dim3(xcd_grid(rows, kHq)), dim3(kCombineThreads), 0, stream, w.part_o, w.part_lse, rows,
                       p.nsplit, out, lse);
    return hipGetLastError();
}

}  // namespace

int attn_num_splits(int rows, int k) { return plan(rows, k).nsplit; }

size_t attn_ws_bytes(int rows, int k) {
    if (plan(rows, k).nsplit == 1) return 0;
    return part_o_bytes(rows, k) + part_lse_bytes(rows, k);
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* kv, int64_t kv_bstride, const int32_t* idx, int B, int T,
                       int L, int k, float sm_scale, uint16_t* out, float* lse, void* ws, hipStream_t stream) {
    return launch_attn_impl<false>(q, kv, kv_bstride, idx, B, T, L, k, sm_scale, out, lse, ws, stream);
}

hipError_t launch_attn_fp8(const uint16_t* q, const uint8_t* kv, int64_t kv_bstride, const int32_t* idx, int B,
                           int T, int L, int k, float sm_scale, uint16_t* out, float* lse, void* ws,
                           hipStream_t stream) {
    return launch_attn_impl<true>(q, kv, kv_bstride, idx, B, T, L, k, sm_scale, out, lse, ws, stream);
}

}  // namespace dsa
