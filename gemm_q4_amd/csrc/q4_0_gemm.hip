// Prefill Q4_0 product on the matrix cores: y[n x out] = x . W^T for large n.
//
// The compute-bound case (goinfer primer ch. 10, "What the kernels are": GEMM
// is prefill's workhorse; golem reads prompts in passes of up to 512
// positions, golem README "Reading a prompt on the card").
//
// Instruction: v_mfma_f32_32x32x16_f16.  On gfx950 it retires twice the
// flops per cycle of v_mfma_f32_16x16x32_f16, and each issue leaves about
// four VALU slots free; the weight decode costs 14 VALU operations per 8
// weights, so every decoded B fragment is reused by four MFMAs (the wave's
// 128 activation rows).
//
// Tile: a workgroup computes 128 activation rows x 128 weight rows with
// eight waves, two per SIMD.  Wave (wn, wk) owns weight rows [32 wn, 32 wn
// + 32) of the tile, all 128 activation rows, and blocks 2 wk, 2 wk + 1 of
// every 4-block group (128 k) of the workgroup's K slice: 4 accumulators of
// 32 x 32.  No weight fragment is decoded twice in a workgroup, and while
// one wave of a SIMD waits (on LDS, on the step barrier) the other's
// products keep the matrix unit busy.  At the end the two K halves are
// summed through LDS.  Build options keep the two earlier splits: four
// waves, one per SIMD, each 128 activation rows x 64 weight rows (each A
// fragment feeds two products), and eight waves splitting the activation
// rows in two (64 x 64 per wave, every weight fragment decoded twice).
//
// Operands of one MFMA (K = 16, half a Q4_0 block):
//   A: lane l = 32h + m holds activation row m of its 32-row sub-tile at
//      k = 16ks + 8h .. +7 of the group (natural order, 16 bytes).  The
//      group's x tile (128 rows x 128 k, binary16) is staged in LDS, four
//      groups ahead (direct copies from global memory for binary16 x;
//      float32 x goes through registers and is rounded to binary16).
//   B: lane l = 32h + c holds weight row c of a 32-row sub-tile at the same
//      k.  k = 8h..8h+7 of a block are the low nibbles of code bytes
//      8h..8h+7, k = 16+8h.. their high nibbles, so the lane loads the
//      repacked words of quarters 2h and 2h+1 (4 bytes per block) and one
//      word pair yields the B fragments of both K halves of a block.  Each
//      value is exact q - 8 times d, rounded once to binary16.
//   D: lane l holds weight row l%32 and activation rows 8(i/4) + 4h + i%4.
//
// Work split: whole 128 x 128 tiles for every full pass over the compute
// units (256 on MI355X); the tiles of the last, partial pass are cut along K into slices
// that spread over all compute units, their partial tiles parked in a
// workspace and added in slice order by a second kernel (deterministic).
// Consecutive workgroup ids are dealt to the dies (eight) in turn; the ids are
// permuted so that each die takes a contiguous run of tiles in which the M
// blocks of one N block are adjacent, and its L2 serves their shared words.
#include <type_traits>

#include "q4_0_device.h"
#include "q4_0_dma.h"
#include "q4_0_internal.h"

namespace q4 {


constexpr int kGemmBM = 128;                 // activation rows per workgroup
constexpr int kGemmBN = 128;                 // weight rows per workgroup
// Waves per workgroup: 8 (two per SIMD) or 4 (one per SIMD, each wave 128
// activation rows x 64 weight rows x half of K).  Measured on MI355X (graph
// replay, three alternating runs): FFN-up 512 x 2560 . (9728 x 2560)^T
// 39.0 us with eight waves splitting the weight rows against 40.1 us with
// four, FFN-down 36.0 against 37.0 us; eight waves splitting the activation
// rows instead took 43.0 / 40.2 us.
#ifndef Q4_GEMM_WAVES
#define Q4_GEMM_WAVES 8
#endif
constexpr int kGemmWaves = Q4_GEMM_WAVES;
// Partial tiles of the K slices stored with non-temporal stores (1) or plain
// stores (0: they stay in the caches for the reduction kernel that follows).
#ifndef Q4_GEMM_NT_PARTIALS
#define Q4_GEMM_NT_PARTIALS 1
#endif
static_assert(kGemmWaves == 4 || kGemmWaves == 8, "4 or 8 waves");
constexpr int kThreads = kGemmWaves * 64;
// With eight waves, split the tile's weight rows four ways (1) or its
// activation rows two ways (0: each wave 64 x 64 x half of K).
#ifndef Q4_GEMM_NSPLIT
#define Q4_GEMM_NSPLIT 1
#endif
constexpr bool kNSplit = Q4_GEMM_NSPLIT && kGemmWaves == 8;
constexpr int kGemmMHalves = kNSplit ? 1 : kGemmWaves / 4;   // waves along the activation rows
constexpr int kGemmMSub = kGemmBM / 32 / kGemmMHalves;  // 32-row sub-tiles per wave
constexpr int kNi = kNSplit ? 1 : 2;                     // 32-row weight sub-tiles per wave
constexpr int kWaveCols = 32 * kNi;                      // weight rows per wave
constexpr int kMfmaPerK = kGemmMSub * kNi;               // products per K-step
constexpr int kStepBytes = kGemmBM * 128 * 2;  // one step's x tile: 32 KB
constexpr int kPiecesPerThread = kStepBytes / 16 / kThreads;  // 8 or 4
constexpr int kPiecesPerPart = (kPiecesPerThread + 2) / 3;    // x pieces in parts 0..2
constexpr int kTilesPerWave = 8 / kGemmWaves;     // 16-row code tiles a wave copies
constexpr int kXBytes = kStepBytes;              // x part of a stage
constexpr int kWBytes = 8 * kGroupCodeBytes;      // code words of the 8 repacked tiles
constexpr int kSBytes = kGemmWaves * 1024;        // their scales: a 1 KB slot per wave
constexpr int kStageBytes = kXBytes + kWBytes + kSBytes;   // 44 or 48 KB
constexpr int kStages = 3;                        // LDS ring: 132 or 144 KB
constexpr int kCopies = kPiecesPerThread + kTilesPerWave + 1;  // copies per wave per step
constexpr int kCopyParts012 = kPiecesPerThread + 1;   // of them in parts 0..2 of a step
constexpr int kTileStride = 136;                  // epilogue tile row, floats
constexpr int kEpiBytes = kGemmBM * kTileStride * 4;   // 68 KB
constexpr int kGemmLds = kStages * kStageBytes > kEpiBytes ? kStages * kStageBytes : kEpiBytes;
static_assert(kGemmLds <= 160 * 1024, "LDS of one workgroup");

struct GemmArgs {
    const uint8_t *packed;
    const void *x;
    float *y;
    float *part;          // partial tiles of the split work, 128 x 128 each
    int64_t code_base;    // byte offset of the code stream
    int n, out, in;
    int g4, tiles;        // layout: groups per row, 16-row tiles
    int nm, nn;           // M blocks, N blocks (tile t: M block t % nm, N block t / nm)
    int full;             // tiles 0 .. full-1 are computed whole
    int rem, split, gps;  // the rem other tiles: split K slices of gps groups each
    int dies;             // dies (L2 domains) the ids are dealt over
    int die_full, die_split;  // permute ids per die in each part
};

// 8 consecutive float32 activations (zeros when !ok), and their binary16 form
struct X8 {
    float4 a, b;
};
__device__ __forceinline__ X8 load_x8(const float *__restrict__ src, bool ok) {
    X8 v = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (ok) {
        v.a = *reinterpret_cast<const float4 *>(src);
        v.b = *reinterpret_cast<const float4 *>(src + 4);
    }
    return v;
}
__device__ __forceinline__ u4_t to_half8(const X8 &v) {
    u4_t h;
    h[0] = as_u32(h2_t{(_Float16)v.a.x, (_Float16)v.a.y});
    h[1] = as_u32(h2_t{(_Float16)v.a.z, (_Float16)v.a.w});
    h[2] = as_u32(h2_t{(_Float16)v.b.x, (_Float16)v.b.y});
    h[3] = as_u32(h2_t{(_Float16)v.b.z, (_Float16)v.b.w});
    return h;
}




template <typename XT>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];   // kGemmLds bytes
    constexpr bool kDma = sizeof(XT) == 2;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, c = lane & 31;
    const Magic mg = pinned_magic();

    // ---- which tile and K range ---------------------------------------------
    // Ids below `full` take whole tiles; the others take K slices of the
    // remaining tiles (piece q = slice * rem + tile - full, so consecutive
    // pieces share a slice of the weights).  Within each part, consecutive
    // ids are dealt to the eight dies in turn; they are permuted so each die
    // takes a contiguous run, whose tiles share weight words in its L2.
    const int id = blockIdx.x;
    int tile, gs0, gs1, piece = -1;
    if (id < a.full) {
        tile = a.die_full ? (id % a.dies) * (a.full / a.dies) + id / a.dies : id;
        gs0 = 0;
        gs1 = a.g4;
    } else {
        const int np = a.rem * a.split;
        int q = id - a.full;
        if (a.die_split) q = (q % a.dies) * (np / a.dies) + q / a.dies;
        piece = q;
        tile = a.full + q % a.rem;
        gs0 = (q / a.rem) * a.gps;
        gs1 = gs0 + a.gps < a.g4 ? gs0 + a.gps : a.g4;
    }
    const int mb = tile % a.nm;
    const int nb = tile / a.nm;
    const int wn = kNSplit ? (wave & 3) : (wave & 1);
    const int wk = kNSplit ? (wave >> 2) & 1 : (wave >> 1) & 1;
    const int wm = kNSplit ? 0 : wave >> 2;
    const int m0 = mb * kGemmBM;
    const int nsteps = gs1 - gs0;
    const XT *__restrict__ x = (const XT *)a.x;

    // ---- copies of one step into a stage -----------------------------------
    // x: 128 activation rows x 16 chunks of 8 binary16 (chunk q = k 8q..8q+7
    // of the group), row-major, the chunks of row r XOR-swizzled: chunk q of
    // row r sits in slot r * 16 + (q ^ (r & 15)).  A copy instruction fills 64
    // consecutive slots = 4 whole rows (coalesced reads); the fragment reads
    // hit 16 distinct slot columns per 16 lanes (no bank conflict).  Wave w
    // fills rows R w .. R w + R - 1 (R = 4 x pieces per thread), copy i rows
    // R w + 4 i + lane / 16.  Rows
    // past n repeat row n - 1 (a D row depends only on its own A row, and
    // those rows are not stored); in a group that runs past in, k >= in is
    // zero.
    // W: the group's code words of the tile's 8 repacked 16-row tiles (1 KB
    // each, as stored) and their scales; wave w copies T = 8 / waves tiles
    // Tw .. Tw + T - 1 and their scales (lanes 0..8T-1 carry the 128 T scale
    // bytes, the other lanes repeat them into the rest of the wave's 1 KB
    // scale slot, so the copy needs no branch).  Tiles past the matrix read
    // the last tile (their scales are forced to zero when used).
    uint32_t xoff[kPiecesPerThread];
#pragma unroll
    for (int i = 0; i < kPiecesPerThread; ++i) {
        const int r = 4 * kPiecesPerThread * wave + 4 * i + (lane >> 4);
        const int q = (lane & 15) ^ (r & 15);
        const int rr = m0 + r < a.n ? r : a.n - 1 - m0;
        xoff[i] = ((uint32_t)rr * a.in + 8 * q) * (uint32_t)sizeof(XT);
    }
    const XT *xbase = x + (int64_t)m0 * a.in;
    const int t0 = nb * (kGemmBN / kTileRows);               // first repacked tile
    int tw[kTilesPerWave];
#pragma unroll
    for (int u = 0; u < kTilesPerWave; ++u) {
        const int t = t0 + kTilesPerWave * wave + u;
        tw[u] = t < a.tiles ? t : a.tiles - 1;
    }
    const int ts = tw[((lane >> 3) & 1) % kTilesPerWave];
    const uint32_t soff_copy = (uint32_t)ts * a.g4 * kGroupScaleBytes + (lane & 7) * 16;
    // byte offsets of the lane's code words from a group's first tile (the
    // code stream is below 4 GiB: gemm_supports)
    uint32_t woff_copy[kTilesPerWave];
#pragma unroll
    for (int u = 0; u < kTilesPerWave; ++u)
        woff_copy[u] = (uint32_t)tw[u] * a.g4 * kGroupCodeBytes + lane * 16;

    // part p < 3 of step st's copies: x pieces P p .. P p + P - 1 (binary16
    // x only, P = kPiecesPerPart); code tile u of the wave at part 2 + u; the
    // scales at part 3
    auto fill = [&](int st, auto sg, int part, bool partial) {
        const int j = gs0 + st;
        uint8_t *stage = lds + sg * kStageBytes;
        if constexpr (kDma) {
            uint8_t *xd = stage + wave * (kPiecesPerThread * 1024);
            const uint8_t *src = (const uint8_t *)(xbase + j * 128);
#pragma unroll
            for (int i = 0; i < kPiecesPerThread; ++i) {
                if (part > 2 || i < kPiecesPerPart * part || i >= kPiecesPerPart * (part + 1))
                    continue;
                if (partial) {
                    // a group running past in: those lanes read a zero piece
                    const int r = 4 * kPiecesPerThread * wave + 4 * i + (lane >> 4);
                    const int q = (lane & 15) ^ (r & 15);
                    const void *p = j * 128 + 8 * q < a.in ? (const void *)(src + xoff[i])
                                                           : (const void *)&kZeroPiece;
                    dma16(p, xd + i * 1024);
                } else {
                    dma16_at(src, xoff[i], xd + i * 1024);
                }
            }
        }
        const uint8_t *cgroup = a.packed + a.code_base + (int64_t)j * kGroupCodeBytes;
#pragma unroll
        for (int u = 0; u < kTilesPerWave; ++u)
            if (part == 2 + u)
                dma16_at(cgroup, woff_copy[u], stage + kXBytes + (kTilesPerWave * wave + u) * 1024);
        if (part == 3)
            dma16_at(a.packed + (int64_t)j * kGroupScaleBytes, soff_copy,
                     stage + kXBytes + kWBytes + wave * 1024);
    };
    X8 xp[kDma ? 1 : kPiecesPerThread];
    auto fetch = [&](int st) {                     // register path (float32 x): load
        if constexpr (!kDma) {
            const int j = gs0 + st;
            const uint8_t *src = (const uint8_t *)(xbase + j * 128);
#pragma unroll
            for (int i = 0; i < kPiecesPerThread; ++i) {
                const int r = 4 * kPiecesPerThread * wave + 4 * i + (lane >> 4);
                const int q = (lane & 15) ^ (r & 15);
                const bool ok = j * 128 + 8 * q < a.in;
                xp[i] = load_x8((const float *)(src + xoff[i]), ok);
            }
        }
    };
    auto park = [&](auto sg) {                     // register path: convert, write the stage
        if constexpr (!kDma) {
            uint8_t *xd = lds + sg * kStageBytes + wave * (kPiecesPerThread * 1024) +
                          lane * 16;
#pragma unroll
            for (int i = 0; i < kPiecesPerThread; ++i)
                *reinterpret_cast<u4_t *>(xd + i * 1024) = to_half8(xp[i]);
        }
    };
    // fragment read offsets: lane (h, m) reads row 32 mi + m, chunk 2 ks + h
    uint32_t aoff[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) aoff[ks] = c * 256 + 16 * ((2 * ks + h) ^ (c & 15));
    // weight words of the lane in a stage: sub-tile ni = rows W wn + 32 ni + c
    // (W = kWaveCols weight rows per wave) = tile (W / 16) wn + 2 ni + c / 16,
    // row c % 16; quarter 2h (+1: 256 bytes on),
    // blocks 2 wk, 2 wk + 1 (8 bytes); their scales (4 bytes) in the slot of
    // the wave that copied the tile (128 bytes per tile in the slot)
    uint32_t woff[kNi], sgoff[kNi];
    bool wvalid[kNi];
#pragma unroll
    for (int ni = 0; ni < kNi; ++ni) {
        const int tl = (kWaveCols / 16) * wn + 2 * ni + (c >> 4);
        wvalid[ni] = t0 + tl < a.tiles;
        woff[ni] = kXBytes + tl * 1024 + ((2 * h) * 16 + (c & 15)) * 16 + 8 * wk;
        sgoff[ni] = kXBytes + kWBytes + (tl / kTilesPerWave) * 1024 + (tl % kTilesPerWave) * 128 +
                    (c & 15) * 8 + 4 * wk;
    }

    f16x_t acc[kGemmMSub][kNi];
#pragma unroll
    for (int mi = 0; mi < kGemmMSub; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNi; ++ni)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mi][ni][v] = 0.0f;

    const h2_t off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2_t off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};

    // ---- operands ------------------------------------------------------------
    // The wave's part of a group: blocks 2wk, 2wk+1 = K-steps ks = 4wk+kq,
    // kq = 0..3.  K-step kq uses A from the stage and, per sub-tile, B = low
    // (kq even) or high (kq odd) nibbles of block 2wk + kq / 2.
    u2_t w0[kNi], w1[kNi];                                   // code words of the step
    uint32_t sc[kNi];                                        // their scales
    uint32_t p01a[kNi], p23a[kNi], p01b[kNi], p23b[kNi];    // byte-spread words of a block
    h2_t d2[kNi];
    h8_t A[2][kGemmMSub];
    h8_t B[2][kNi];
    auto read_w = [&](auto sg) {
        const uint8_t *stage = lds + sg * kStageBytes;
#pragma unroll
        for (int ni = 0; ni < kNi; ++ni) {
            w0[ni] = *reinterpret_cast<const u2_t *>(stage + woff[ni]);
            w1[ni] = *reinterpret_cast<const u2_t *>(stage + woff[ni] + 256);
            sc[ni] = *reinterpret_cast<const uint32_t *>(stage + sgoff[ni]);
        }
    };
    auto spread = [&](int b) {                              // b: 0 or 1, block 2wk + b
#pragma unroll
        for (int ni = 0; ni < kNi; ++ni) {
            const uint32_t u0 = w0[ni][b], u1 = w1[ni][b];
            p01a[ni] = __builtin_amdgcn_perm(u0, u0, 0x0C010C00u);
            p23a[ni] = __builtin_amdgcn_perm(u0, u0, 0x0C030C02u);
            p01b[ni] = __builtin_amdgcn_perm(u1, u1, 0x0C010C00u);
            p23b[ni] = __builtin_amdgcn_perm(u1, u1, 0x0C030C02u);
            const _Float16 d = wvalid[ni] ? as_h2(sc[ni])[b] : (_Float16)0.0f;
            d2[ni] = h2_t{d, d};
        }
    };
    auto frag = [&](bool hi, int ni) -> h8_t {
        const uint32_t mask = hi ? kMaskHi : kMaskLo;
        const uint32_t magic = hi ? mg.hi : mg.lo;
        const h2_t off = hi ? off_hi : off_lo;
        u4_t b;
        b[0] = as_u32((as_h2((p01a[ni] & mask) | magic) + off) * d2[ni]);
        b[1] = as_u32((as_h2((p23a[ni] & mask) | magic) + off) * d2[ni]);
        b[2] = as_u32((as_h2((p01b[ni] & mask) | magic) + off) * d2[ni]);
        b[3] = as_u32((as_h2((p23b[ni] & mask) | magic) + off) * d2[ni]);
        return __builtin_bit_cast(h8_t, b);
    };
    auto read_a = [&](auto sg, int kq, h8_t (&av)[kGemmMSub]) {
        const uint8_t *stage = lds + sg * kStageBytes;
#pragma unroll
        for (int mi = 0; mi < kGemmMSub; ++mi)
            av[mi] = __builtin_bit_cast(
                h8_t, *reinterpret_cast<const u4_t *>(stage + aoff[4 * wk + kq] +
                                                     (kGemmMSub * wm + mi) * 8192));
    };
    // operands of K-step 0 of step st into buffer 0
    auto prep_first = [&](auto sg) {
        read_w(sg);
        read_a(sg, 0, A[0]);
        spread(0);
#pragma unroll
        for (int ni = 0; ni < kNi; ++ni) B[0][ni] = frag(false, ni);
    };
    // Interleave: one MFMA, then an LDS read and up to four VALU operations.
    // A wave issues in order and each MFMA holds the issue port while the
    // matrix pipe takes it, so only work placed between the products
    // overlaps them; the scheduling groups enforce that order inside the
    // (branch-free) region.
    constexpr int kValuPerMfma = 16 / kGemmMSub;                 // 4 or 8
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < kMfmaPerK; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
            __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);   // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto products = [&](int cur) {
#pragma unroll
        for (int ni = 0; ni < kNi; ++ni)
#pragma unroll
            for (int mi = 0; mi < kGemmMSub; ++mi)
                acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[cur][mi], B[cur][ni],
                                                                     acc[mi][ni], 0, 0, 0);
    };

    // ---- one step --------------------------------------------------------------
    // K-steps 0..2 multiply while preparing K-step kq + 1 and issuing copy
    // parts 0..2 of step st + 2.  Then a wait until step st + 1's copies have
    // landed (its last part was issued one step ago; only parts 0..2 of step
    // st + 2 are newer) and a barrier.  K-step 3 multiplies while issuing
    // part 3 of step st + 2 and preparing K-step 0 of step st + 1.  The
    // barrier also frees stage st for the copies of step st + 3.
    // REQ: step st + 2 exists; PART: its group runs past in; NEXT: st + 1
    // exists.
    // sg: the LDS stage of step st (st mod kStages), a compile-time constant in
    // the unrolled main loop, so every stage address folds into the LDS
    // instructions' offsets.
    auto step = [&](int st, auto sg, auto req_t, auto part_t, auto next_t) {
        constexpr bool REQ = decltype(req_t)::value;
        constexpr bool PART = decltype(part_t)::value;
        constexpr bool NEXT = decltype(next_t)::value;
        const int sg_req = (sg + kStages - 1) % kStages;      // stage of step st + 2
        const int sg_next = (sg + 1) % kStages;               // stage of step st + 1
        if constexpr (REQ && !kDma) fetch(st + kStages - 1);
        // The copies open each region: inline assembly is a scheduling
        // boundary, so copies placed between the products and the operand
        // work would keep the two from interleaving.
#pragma unroll
        for (int kq = 0; kq < 3; ++kq) {
            const int cur = kq & 1;
            if (REQ) fill(st + kStages - 1, sg_req, kq, PART);
            products(cur);
            read_a(sg, kq + 1, A[cur ^ 1]);
            if (kq == 1) spread(1);
#pragma unroll
            for (int ni = 0; ni < kNi; ++ni) B[cur ^ 1][ni] = frag(kq != 1, ni);
            interleave();
        }
        if constexpr (NEXT) {
            if constexpr (REQ) Q4_WAIT_VMCNT(kCopyParts012);
            else Q4_WAIT_VMCNT(0);
            Q4_WAIT_LGKM0();
            __builtin_amdgcn_s_barrier();
        }
        if (REQ) fill(st + kStages - 1, sg_req, 3, PART);
        products(1);
        if constexpr (NEXT) {
            // next step's weight words first, two products while they
            // travel, then the decode between the remaining products
            prep_first(sg_next);
            constexpr int kLead = kGemmMSub / 2;                    // products while words travel
            __builtin_amdgcn_sched_group_barrier(0x100, 3 * kNi, 0);  // DS read: words, scales
            __builtin_amdgcn_sched_group_barrier(0x008, kLead, 0);  // MFMA
#pragma unroll
            for (int i = 0; i < kMfmaPerK - kLead; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read: A
                __builtin_amdgcn_sched_group_barrier(0x002, 24 * kNi / (kMfmaPerK - kLead), 0);  // VALU
            }
            __builtin_amdgcn_sched_barrier(0);
        } else {
            interleave();
        }
        if constexpr (REQ && !kDma) park(sg_req);
    };

    // ---- pipeline ------------------------------------------------------------
    // Steps 0 and 1 are requested up front, step st + 2 during step st; all
    // requests are direct copies into LDS whose counts are managed here (the
    // loop holds no loads into registers, so the compiler adds no waits).
    // The float32 path stages x through registers instead: loaded at the top
    // of step st, converted and written at its end.
    for (int p = 0; p < kStages - 1 && p < nsteps; ++p) {
#pragma unroll
        for (int part = 0; part < 4; ++part) fill(p, p, part, (gs0 + p) * 128 + 128 > a.in);
        if constexpr (!kDma) { fetch(p); park(p); }
    }
    if (nsteps > 1) Q4_WAIT_VMCNT(kCopies);
    else Q4_WAIT_VMCNT(0);
    Q4_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    prep_first(std::integral_constant<int, 0>());
    // The steady state runs one variant of the step (the next-but-one step
    // exists and its group lies inside the row); the at most three last
    // steps are peeled, so the accumulators keep one register assignment
    // through the loop.
    using T = std::true_type;
    using F = std::false_type;
    const bool last_partial = gs1 * 128 > a.in;              // the slice's last group runs past in
    const int n_main = nsteps - (kStages - 1) - (last_partial ? 1 : 0);
    int st = 0;
    static_assert(kStages == 3, "the main loop is unrolled over three stages");
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    for (; st + kStages <= n_main; st += kStages) {
        step(st, S0(), T(), F(), T());
        step(st + 1, S1(), T(), F(), T());
        step(st + 2, S2(), T(), F(), T());
    }
    for (; st < n_main; ++st) step(st, st % kStages, T(), F(), T());
    if (last_partial && st == nsteps - kStages) { step(st, st % kStages, T(), T(), T()); ++st; }
    if (st == nsteps - 2) { step(st, st % kStages, F(), F(), T()); ++st; }
    if (st == nsteps - 1) { step(st, st % kStages, F(), F(), F()); ++st; }
    Q4_WAIT_VMCNT(0);
    Q4_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();

    // ---- epilogue ------------------------------------------------------------
    // The tile's stores are non-temporal: written once, never read again by
    // this kernel, and issued by all compute units at about the same time
    // (measured in alternating runs: FFN-up 512 x 2560 . (9728 x 2560)^T
    // 42.2-42.8 us against 43.4-43.8 us, FFN-down 39.4-39.7 against 39.7-40.0).
    // The K half wk = 1 writes its sums into a row-major tile in LDS (row
    // stride 136 floats: the two row groups of a write instruction land in
    // disjoint banks); wk = 0 reads them all, adds its own and writes the
    // tile back; then all the waves store whole rows, 16 bytes per lane.
    // Reads before writes: the compiler keeps LDS accesses that may alias in
    // program order, so interleaving them would serialize on LDS latency.
    float *ttile = reinterpret_cast<float *>(lds);           // 128 x 136 floats
    // lane holds tile column W wn + 32 ni + c, tile rows
    // 32 mi + 8 (v / 4) + 4 h + v % 4
    auto tix = [&](int mi, int ni, int v) {
        return (32 * (kGemmMSub * wm + mi) + 8 * (v >> 2) + 4 * h + (v & 3)) * kTileStride +
               kWaveCols * wn + 32 * ni + c;
    };
    if (wk == 1) {
#pragma unroll
        for (int mi = 0; mi < kGemmMSub; ++mi)
#pragma unroll
            for (int ni = 0; ni < kNi; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) ttile[tix(mi, ni, v)] = acc[mi][ni][v];
    }
    Q4_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    if (wk == 0) {
        float other[kGemmMSub][kNi][16];
#pragma unroll
        for (int mi = 0; mi < kGemmMSub; ++mi)
#pragma unroll
            for (int ni = 0; ni < kNi; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) other[mi][ni][v] = ttile[tix(mi, ni, v)];
#pragma unroll
        for (int mi = 0; mi < kGemmMSub; ++mi)
#pragma unroll
            for (int ni = 0; ni < kNi; ++ni)
#pragma unroll
                for (int v = 0; v < 16; ++v) ttile[tix(mi, ni, v)] = acc[mi][ni][v] + other[mi][ni][v];
    }
    Q4_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    const int n0 = nb * kGemmBN;
    if (piece >= 0) {
        // a K slice: the whole 128 x 128 partial tile, row-major, to the workspace
        float *dst = a.part + (int64_t)piece * kGemmBM * kGemmBN;
#pragma unroll 4
        for (int it = 0; it < kGemmBM * kGemmBN / 4 / kThreads; ++it) {
            const int e = it * kThreads + tid;                 // float4 index in the tile
            const int row = e >> 5, col = (e & 31) * 4;
            const f4_t v = *reinterpret_cast<const f4_t *>(ttile + row * kTileStride + col);
            f4_t *d = reinterpret_cast<f4_t *>(dst + row * kGemmBN + col);
#if Q4_GEMM_NT_PARTIALS
            __builtin_nontemporal_store(v, d);
#else
            *d = v;
#endif
        }
        return;
    }
    const bool full_cols = n0 + kGemmBN <= a.out && (a.out & 3) == 0;
#pragma unroll 4
    for (int it = 0; it < kGemmBM * kGemmBN / 4 / kThreads; ++it) {
        const int e = it * kThreads + tid;                     // float4 index in the tile
        const int row = e >> 5, col = (e & 31) * 4;
        if (m0 + row >= a.n) continue;
        const float4 v = *reinterpret_cast<const float4 *>(ttile + row * kTileStride + col);
        float *yp = a.y + (int64_t)(m0 + row) * a.out + n0 + col;
        if (full_cols) {
            __builtin_nontemporal_store(__builtin_bit_cast(f4_t, v), reinterpret_cast<f4_t *>(yp));
        } else {
            const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (n0 + col + q < a.out) yp[q] = vv[q];
        }
    }
}

// y of the split tiles = sum of their K slices' partial tiles, in slice order.
constexpr int kReduceBatch = 8;   // slice loads in flight per thread
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float *__restrict__ part,
                                                          float *__restrict__ y, int n, int out,
                                                          int nm, int full, int rem, int split) {
    const int64_t count = (int64_t)rem * kGemmBM * kGemmBN / 4;   // float4 items
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < count; e += stride) {
        const int r = (int)(e / (kGemmBM * kGemmBN / 4));
        const int local = (int)(e % (kGemmBM * kGemmBN / 4)) * 4;
        const int row = local / kGemmBN, col = local % kGemmBN;
        const int t = full + r;
        const int grow = (t % nm) * kGemmBM + row, gcol = (t / nm) * kGemmBN + col;
        if (grow >= n) continue;
        // the slices' loads are issued in batches (indices past the last
        // slice re-read it and are not added), then added in slice order
        float4 s4 = {0.f, 0.f, 0.f, 0.f};
        for (int q0 = 0; q0 < split; q0 += kReduceBatch) {
            float4 v[kReduceBatch];
#pragma unroll
            for (int b = 0; b < kReduceBatch; ++b) {
                const int q = q0 + b < split ? q0 + b : split - 1;
                v[b] = *reinterpret_cast<const float4 *>(
                    part + ((int64_t)q * rem + r) * kGemmBM * kGemmBN + local);
            }
#pragma unroll
            for (int b = 0; b < kReduceBatch; ++b) {
                const bool on = q0 + b < split;
                s4.x += on ? v[b].x : 0.f;
                s4.y += on ? v[b].y : 0.f;
                s4.z += on ? v[b].z : 0.f;
                s4.w += on ? v[b].w : 0.f;
            }
        }
        float *yp = y + (int64_t)grow * out + gcol;
        const float vv[4] = {s4.x, s4.y, s4.z, s4.w};
        if (gcol + 4 <= out && (out & 3) == 0) {
            *reinterpret_cast<float4 *>(yp) = s4;
        } else {
            for (int q = 0; q < 4; ++q)
                if (gcol + q < out) yp[q] = vv[q];
        }
    }
}

// Work split: whole tiles for as many full passes over the device's compute
// units as the tile count allows; the remaining tiles (a partial pass) are
// cut along K into as many slices as spread them over the compute units, each
// slice at least kMinSliceGroups groups, and a second kernel adds the slices.
constexpr int kMinSliceGroups = 4;
struct GemmPlan {
    int nm, nn, full, rem, split, gps;
    int64_t wgs;
};

static GemmPlan gemm_plan(int64_t n, int64_t out, int64_t in) {
    const Layout L(out, in);
    const int64_t cus = device_shape().cus;
    GemmPlan p;
    p.nm = (int)((n + kGemmBM - 1) / kGemmBM);
    p.nn = (int)((out + kGemmBN - 1) / kGemmBN);
    const int64_t tiles = (int64_t)p.nm * p.nn;
    const int64_t rem = tiles % cus;
    int64_t split = rem > 0 ? cus / rem : 1;
    const int64_t max_split = L.g4 / kMinSliceGroups;
    if (split > max_split) split = max_split;
    if (split < 2) {
        p.full = (int)tiles;
        p.rem = 0;
        p.split = 1;
        p.gps = (int)L.g4;
    } else {
        p.full = (int)(tiles - rem);
        p.rem = (int)rem;
        p.gps = (int)((L.g4 + split - 1) / split);
        p.split = (int)((L.g4 + p.gps - 1) / p.gps);
    }
    p.wgs = (int64_t)p.full + (int64_t)p.rem * p.split;
    return p;
}

size_t gemm_workspace_bytes(int64_t n, int64_t out, int64_t in) {
    const GemmPlan p = gemm_plan(n, out, in);
    return (size_t)p.rem * p.split * kGemmBM * kGemmBN * sizeof(float);
}

bool gemm_supports(int64_t n, int64_t out, int64_t in, int x_f16) {
    (void)x_f16;
    if (n < 1 || out < 1 || in < 32) return false;
    // the copies address the code stream with 32-bit offsets from each group
    if (Layout(out, in).total_bytes() >= ((int64_t)1 << 32)) return false;
    if (n * out > 0x7fffffff || n * in > ((int64_t)1 << 40)) return false;
    const GemmPlan p = gemm_plan(n, out, in);
    return p.wgs <= 0x7fffffff && gemm_workspace_bytes(n, out, in) <= kWorkspaceBytes;
}

hipError_t launch_gemm(const void *packed, const void *x, int x_f16, float *y, int64_t n,
                       int64_t out, int64_t in, void *ws, hipStream_t stream) {
    const Layout L(out, in);
    const GemmPlan p = gemm_plan(n, out, in);
    GemmArgs a;
    a.packed = (const uint8_t *)packed;
    a.x = x;
    a.y = y;
    a.part = p.rem > 0 ? (float *)ws : nullptr;
    a.code_base = L.scale_bytes();
    a.n = (int)n;
    a.out = (int)out;
    a.in = (int)in;
    a.g4 = (int)L.g4;
    a.tiles = (int)L.tiles;
    a.nm = p.nm;
    a.nn = p.nn;
    a.full = p.full;
    a.rem = p.rem;
    a.split = p.split;
    a.gps = p.gps;
    a.dies = device_shape().dies;
    a.die_full = (p.full > 0 && p.full % a.dies == 0) ? 1 : 0;
    a.die_split = (p.rem > 0 && (p.rem * p.split) % a.dies == 0) ? 1 : 0;
    const dim3 grid((unsigned)p.wgs), block(kThreads);
    const size_t lds = (size_t)kGemmLds;
    if (x_f16)
        hipLaunchKernelGGL(gemm_kernel<_Float16>, grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL(gemm_kernel<float>, grid, block, lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.rem == 0) return e;
    const int64_t count = (int64_t)p.rem * kGemmBM * kGemmBN / 4;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)grid_for(count, 256)), dim3(256), 0,
                       stream, (const float *)a.part, y, (int)n, (int)out, p.nm, p.full, p.rem,
                       p.split);
    return hipGetLastError();
}

}  // namespace q4
