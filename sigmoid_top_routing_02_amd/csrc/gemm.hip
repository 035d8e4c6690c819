// Grouped block-scaled FP8 GEMM for the expert FFNs (and, with one group, the
// dense block-scaled GEMM).
//
// "DeepSeek-V3 Technical Report" notes (learn.ifs.name), FP8-accumulation
// paragraph: the tensor-core accumulation of FP8 products is promoted to FP32
// every 128 elements of the inner dimension, and the per-group scales are
// applied there.  On gfx950 one v_mfma_f32_16x16x128_f8f6f4 covers exactly one
// 128-wide slice, so every slice is one MFMA into a fresh FP32 accumulator and
// the scaled sum over slices is an FP32 FMA chain on the VALU:
//     acc = fma(P_j, a_scale[m,j] * b_scale[n/128,j], acc)
// (FP8-tiling paragraph: A is scaled per 1x128 tile, B per 128x128 block.)
//
// Tiling (CDNA4): block tile 128 (M) x 256 (N) (32 x 256 for groups of a few
// rows), one 128-byte K slice per pipeline stage, 8 wave64s in a 2 x 4 grid
// with a 64 x 64 wave tile (4 x 4 MFMA tiles of 16x16), two waves per SIMD.
// Inside a tile the two halves of the workgroup run a phase apart (see the
// kernel): on each SIMD one wave multiplies from registers while the other
// reads the next fragments from LDS and issues DMAs.
//
// Data movement: A rows are gathered through a_row_index (the dispatch
// permutation), so activations are never materialised in expert order.  A, B
// and the A scales of each slice go global -> LDS by buffer_load ... lds (no
// VGPR staging) into a 3-stage ring; LDS rows are 128 bytes with the 16-byte
// chunks of each row permuted (see swz) so that fragment reads are free of
// bank conflicts.  The A scales are first gathered into GEMM row order and
// made slice-major in the workspace (one slice of a tile's scales is one
// contiguous 512-byte run); the B scales of the tile reach LDS once per tile, by
// DMA like the operands.
//
// Schedule: persistent, one block per CU.  A device-built tile list (exclusive
// scan of ceil(rows_g / BM) per group, then one record per tile) fixes the
// order; each XCD takes its share of the list through an atomic counter.  The
// host only needs the total row count.
//
// Epilogues: FP32 store; SwiGLU (B rows interleaved gate/up per 128-row
// block, so one N tile holds the gate and up columns of the same 128 h
// columns); SwiGLU + 1x128 E4M3 re-quantisation of h, whose row maximum over
// the tile's 128 h columns is reduced across the N-waves in LDS.
#include <atomic>
#include <type_traits>

#include "device_math.h"
#include "kernels.h"
#include "moe_fp8.h"

namespace moe {
namespace {

constexpr int BN = 256;
constexpr int BK = 128;                       // one scale slice
constexpr int NWAVES = 8;
constexpr int NT = 64 * NWAVES;
constexpr int GROUP_M = 8;                    // row tiles per L2-sharing group
constexpr int B_BYTES = BN * BK;              // 32 KiB
constexpr int A_MAX_BYTES = 128 * BK;         // A stage buffer (largest row tile)
constexpr int MAX_SLICES = 128;               // K <= 16384

// Row-tile variants: 128 rows (2 x 4 waves of 64 x 64) for well-filled groups,
// 32 rows (1 x 8 waves of 32 x 32) for groups of a few rows (decode), where a
// 128-row tile would spend most MFMA work on padding.  (A 256-row tile would
// halve the B traffic per flop, but 8 waves of 128 x 64 need more than the
// 256 VGPRs a wave can address once the per-slice FP32 partials are counted.)
template <int BM_>
struct Cfg {
    static constexpr int BM = BM_;
    static constexpr int WAVES_M = BM_ >= 64 ? BM_ / 64 : 1;
    static constexpr int WAVES_N = NWAVES / WAVES_M;
    static constexpr int WROWS = BM_ / WAVES_M;           // rows per wave
    static constexpr int MI = WROWS / 16;                  // MFMA row tiles per wave
    static constexpr int WN_COLS = BN / WAVES_N;           // columns per wave
    static constexpr int NI = WN_COLS / 16;                // MFMA column tiles per wave
    static constexpr int A_INSTR = BM_ * BK / 1024;        // 1 KiB DMAs per A copy
    static constexpr int A_COPIES = A_INSTR >= NWAVES ? 1 : NWAVES / A_INSTR;
    static constexpr int A_DMA = A_INSTR * A_COPIES / NWAVES;
    static constexpr int B_DMA = B_BYTES / 1024 / NWAVES;
    static constexpr int DMA_PER_STAGE = A_DMA + B_DMA + 1;   // + one A-scale DMA
    static constexpr int NSTAGES = 3;
    // Cache policy of the B (weight) DMAs.  32-row tiles serve groups of a few
    // rows, where each weight tile is streamed about once: non-temporal loads
    // keep the stream from evicting lines that are re-read (measured 7-9%
    // faster on the decode-shaped GEMMs).  128-row tiles re-read B across row
    // tiles and lose 10% or more with the hint.
    static constexpr int B_AUX = BM_ == 32 ? 2 : 0;
    static_assert(A_INSTR * A_COPIES * 1024 <= A_MAX_BYTES, "A stage too small");
    static_assert(B_DMA % 2 == 0, "B DMA offsets come in swizzle-parity pairs");
    static_assert(DMA_PER_STAGE == 6 || DMA_PER_STAGE == 7, "stage barrier waits for vmcnt(6|7)");
};

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

struct GemmArgs {
    const uint8_t* a_q;
    const float* a_sT;            // A scales slice-major: [K/128][M_total], in GEMM row order
    uint32_t sa_stride;           // M_total * 4: bytes from one slice's scales to the next
    const int32_t* a_rows;
    const int32_t* group_offset;
    const int32_t* tile_start;
    int32_t* counters;            // [8] next tile of each XCD's share, zeroed by the tile map
    const int4* tiles;            // per tile of the sequence: {group, first row, rows, first column}
    int G;
    const uint8_t* b_q;
    const float* b_s;
    int N;
    int K;
    float* out;
    uint8_t* out_q;
    float* out_s;
    // K-grouped launches only (the weight gradients): group g's inner dimension
    // is its own [kb_start[g], kb_start[g+1]) 128-blocks; its A ([group_rows, Kg]
    // row-major, 1x128 scales [group_rows, Kg/128]) starts at block kb_start[g]
    // of a_q / a_sT, its B ([N, Kg], 128x128 scales [N/128, Kg/128] in rows of
    // b_cs blocks) at that block of b_q / b_s.
    const int32_t* kb_start;
    int group_rows;
    int b_cs;
};

// The three pipeline stages are separate LDS objects and every access names
// its stage at compile time, so the compiler can see that reading one stage
// does not alias the DMA still filling another (it would otherwise wait for
// every outstanding DMA before each LDS read).
__shared__ __attribute__((aligned(1024))) char g_a0[A_MAX_BYTES];
__shared__ __attribute__((aligned(1024))) char g_a1[A_MAX_BYTES];
__shared__ __attribute__((aligned(1024))) char g_a2[A_MAX_BYTES];
__shared__ __attribute__((aligned(1024))) char g_b0[B_BYTES];
__shared__ __attribute__((aligned(1024))) char g_b1[B_BYTES];
__shared__ __attribute__((aligned(1024))) char g_b2[B_BYTES];
// A scales of a slice: wave w DMAs rows 64w .. 64w+63 of the tile into floats
// 64w .. 64w+63 (the waves past the tile's rows issue a DMA that touches no
// memory, so every wave issues the same count); row r < BM is at float r.
__shared__ __attribute__((aligned(16))) float g_sa0[64 * NWAVES];
__shared__ __attribute__((aligned(16))) float g_sa1[64 * NWAVES];
__shared__ __attribute__((aligned(16))) float g_sa2[64 * NWAVES];
__shared__ __attribute__((aligned(16))) float g_bscale[2 * MAX_SLICES];
static_assert(MAX_SLICES == 128, "four 64-lane DMAs fill the B-scale table");


template <int ST, int BM_>
__device__ __forceinline__ char* a_buf() {
    if constexpr (ST == 0) return g_a0;
    else if constexpr (ST == 1) return g_a1;
    else return g_a2;
}
template <int ST>
__device__ __forceinline__ char* b_buf() {
    if constexpr (ST == 0) return g_b0;
    else if constexpr (ST == 1) return g_b1;
    else return g_b2;
}
template <int ST>
__device__ __forceinline__ float* sa_buf() {
    if constexpr (ST == 0) return g_sa0;
    else if constexpr (ST == 1) return g_sa1;
    else return g_sa2;
}

template <int V>
struct IC { static constexpr int value = V; };

// Buffer resource (gfx9 family descriptor word 3); out-of-range offsets read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
// global -> LDS DMA: lane l's `size` bytes land at lds + l*size (lds is wave-uniform).
// AUX is the cache-policy operand; 2 sets the non-temporal bit (gfx950 "nt").
template <int AUX = 0>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, AUX);
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, soff, 0, 0);
}

// LDS tiles hold 128-byte rows; the 16-byte chunk c of row r sits in slot
// c ^ (r & 7) ^ ((r >> 3) & 1).  A fragment read (ds_read_b128) has the 16
// lanes of a group on 16 consecutive rows at one chunk index.  Measured on
// gfx950, such a read runs at full LDS rate only if every 8 consecutive lanes
// hit 8 distinct slots and the 16 lanes cover each (row parity, slot) pair
// once; this swizzle meets both, while c ^ (r & 7) or c ^ ((r >> 1) & 7)
// alone meet one and halve the read rate.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// 32 K-bytes of one MFMA fragment from a swizzled tile.  off0/off1 are the
// lane's byte offsets of its two 16-byte chunks inside a 16-row band
// (row lane%16, chunks 2*kb and 2*kb+1 swizzled); every band starts at a
// multiple of 16 rows, so the swizzle (a function of r mod 16) never changes
// between bands and `band` is a compile-time byte offset.
__device__ __forceinline__ v8i frag(const char* tile, int band, uint32_t off0, uint32_t off1) {
    const uint4 x = *reinterpret_cast<const uint4*>(tile + band + off0);
    const uint4 y = *reinterpret_cast<const uint4*>(tile + band + off1);
    v8i f;
    f[0] = (int)x.x; f[1] = (int)x.y; f[2] = (int)x.z; f[3] = (int)x.w;
    f[4] = (int)y.x; f[5] = (int)y.y; f[6] = (int)y.z; f[7] = (int)y.w;
    return f;
}

// SiLU(z) = z * sigmoid(z), with the hardware exp and reciprocal (not bit-exact
// with any reference; the SwiGLU output is checked against a tolerance).
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Column offset (inside the 256-wide N tile) of MFMA column-tile ni of wave wn.
// SwiGLU waves take WN_COLS/2 gate columns and the matching up columns.
template <int EPI, typename C>
__device__ __forceinline__ int ncol(int wn, int ni) {
    if constexpr (EPI == EPI_STORE_F32) {
        return wn * C::WN_COLS + ni * 16;
    } else {
        constexpr int HALF = C::NI / 2;
        return (ni < HALF) ? (wn * (C::WN_COLS / 2) + ni * 16)
                           : (128 + wn * (C::WN_COLS / 2) + (ni - HALF) * 16);
    }
}

// KG: K-grouped (see GemmArgs).  Every tile then takes its slice count and its
// A, B and scale bases from its group, the A scales are read row-major, and the
// B scales of each slice travel in the scale DMA of wave BM/64 (floats BM and
// BM+1 of the stage's scale buffer) instead of one LDS table per tile, so a
// group's K has no upper bound.
template <int EPI, int BM_, bool KG = false>
__global__ __launch_bounds__(NT) void grouped_gemm_kernel(GemmArgs p) {
    using C = Cfg<BM_>;
    static_assert(!KG || (EPI == EPI_STORE_F32 && BM_ == 128), "K-grouped tiles store FP32 from 128-row tiles");
    constexpr int BM = C::BM, MI = C::MI, NI = C::NI, WAVES_N = C::WAVES_N;
    constexpr int WN_COLS = C::WN_COLS, WROWS = C::WROWS, A_DMA = C::A_DMA, B_DMA = C::B_DMA;
    constexpr int NS = C::NSTAGES;
    // Whether a tile's second slice is issued with its first, before the
    // previous tile's epilogue: when that epilogue leaves stage 1 alone (the
    // SwiGLU epilogues use stage 2 as scratch, the FP32 store of a 32-row tile
    // stages through stage 2 only), so the slice's latency hides behind it.
    constexpr bool EARLY1 = !KG && (EPI != EPI_STORE_F32 || BM_ == 32);
    constexpr int D = C::DMA_PER_STAGE;
    // MFMA operand order.  SwiGLU tiles put B first, so a lane's four results
    // share one output row and one scale (one multiply per row tile instead
    // of four).  FP32-store tiles keep A first (a lane's results are four rows
    // of one column); their output leaves through LDS in whole rows, so the
    // register layout only shapes the LDS writes.
    constexpr bool TR = (EPI != EPI_STORE_F32);
    int K = p.K;          // K-grouped: the current tile's group's (set by setup)
    int ns = K / BK;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;   // wave row / column in the block
    const int kb = lane >> 4;
    const int lr = lane & 15;

    // ---- persistent schedule.  Workgroups go to the 8 XCDs round-robin
    // (block b runs on XCD b % 8) and the grid holds one block per CU.  Each
    // XCD owns one contiguous share of the tile sequence and its blocks take
    // the next tile of that share from a per-XCD counter, so the tiles in
    // flight on an XCD are always neighbours in the sequence.  The sequence
    // walks the groups in order; inside a group it takes chunks of up to
    // GROUP_M row tiles, and inside a chunk the column tile is the slow
    // index: the blocks of an XCD then share the A rows of the chunk and the B
    // columns of one group in the XCD's L2, and never mix two groups' B unless
    // the window straddles a group boundary.  A block asks for its next tile
    // when it starts the current one.
    const int total_tiles = p.tile_start[p.G];
    const int n_tiles = (p.N + BN - 1) / BN;
    const int xcd = blockIdx.x & 7;
    const int total = total_tiles * n_tiles;
    const int share = (total + 7) >> 3;
    __shared__ int s_next;
    struct Tile { int g, m0, rows, n0; };
    auto tile_at = [&](int t) {               // from the list the tile-map kernels built
        const int4 v = p.tiles[t];
        Tile T;                                   // block-uniform: keep it in SGPRs
        T.g = __builtin_amdgcn_readfirstlane(v.x);
        T.m0 = __builtin_amdgcn_readfirstlane(v.y);
        T.rows = __builtin_amdgcn_readfirstlane(v.z);
        T.n0 = __builtin_amdgcn_readfirstlane(v.w);
        return T;
    };
    // the global index of this XCD's tile number tl (-1: none left)
    auto global_tile = [&](int tl) {
        const int t = xcd * share + tl;
        return (tl < share && t < total) ? t : -1;
    };

    // ---- per-tile DMA sources (byte offsets; the slice moves soffset)
    auto a_rsrc = make_rsrc(p.a_q, 0xFFFFFFFFu);
    // every row past M_total (the padding of the last tile) reads scale 0
    auto sa_rsrc = make_rsrc(p.a_sT, p.sa_stride * (uint32_t)ns);
    // A descriptor with no records: every access is out of range, so no memory
    // is touched (the target stage is a spare one).  Past the last slice the
    // pipeline still issues its DMAs through this descriptor, which keeps the
    // instruction stream (and the compiler's wait-count model) identical on
    // every step: no step needs a conservative full drain.
    const auto null_rsrc = make_rsrc(p.a_q, 0u);
    const int nblk_per_g = p.N / 128;
    uint32_t a_off[A_DMA], b_off[2], sa_off = 0;
    uint32_t am_pre[A_DMA];                      // gathered A rows of the next tile's DMA lanes
    __amdgpu_buffer_rsrc_t b_rsrc = null_rsrc;
    __amdgpu_buffer_rsrc_t bs_rsrc = null_rsrc;   // K-grouped: the group's B scales
    const uint8_t* b_group = p.b_q;               // K-grouped: the group's B
    // A-row indices of this lane's A DMAs (the gather)
    auto load_rows = [&](const Tile& T) {
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            // A DMA li = wave*A_DMA + i fills LDS bytes [li*1 KiB, +1 KiB): copy li / A_INSTR
            const int r = ((wave * A_DMA + i) % C::A_INSTR) * 8 + (lane >> 3);
            const int m = T.m0 + min(r, T.rows - 1);
            if constexpr (KG) am_pre[i] = (uint32_t)(m - T.g * p.group_rows);   // row inside the group's A
            else am_pre[i] = p.a_rows ? (uint32_t)p.a_rows[m] : (uint32_t)m;
        }
    };
    auto setup = [&](const Tile& T) {
        if constexpr (KG) {
            const int kb0 = __builtin_amdgcn_readfirstlane(p.kb_start[T.g]);
            ns = __builtin_amdgcn_readfirstlane(p.kb_start[T.g + 1]) - kb0;
            K = ns * BK;
            const int64_t rows_g = p.group_rows;
            a_rsrc = make_rsrc(p.a_q + rows_g * BK * kb0, (uint32_t)(rows_g * K));
            sa_rsrc = make_rsrc(p.a_sT + rows_g * kb0, (uint32_t)(rows_g * ns * 4));
            bs_rsrc = make_rsrc(p.b_s + (int64_t)p.b_cs * kb0, (uint32_t)((p.N / 128) * ns * 4));
            b_group = p.b_q + (int64_t)p.N * BK * kb0;
        }
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int r = ((wave * A_DMA + i) % C::A_INSTR) * 8 + (lane >> 3);
            a_off[i] = am_pre[i] * (uint32_t)K + ((lane & 7) ^ swz(r)) * 16;
        }
        // A scales: the tile's rows are contiguous in the slice-major copy; wave w
        // moves rows 64w .. 64w+63 (waves past the tile's rows move nothing)
        if constexpr (KG) {
            // waves below BM/64: rows of the group's row-major A scales; wave
            // BM/64, lanes 0 and 1: the tile's two B-scale blocks (the second
            // clamped when N % 256 == 128); every other lane reads past the end
            if (wave * 64 < BM)
                sa_off = (uint32_t)((T.m0 - T.g * p.group_rows) + wave * 64 + lane) * (uint32_t)ns * 4u;
            else
                sa_off = lane < 2 ? (uint32_t)min(T.n0 / 128 + lane, p.N / 128 - 1) * (uint32_t)ns * 4u
                                  : 0x80000000u;
            b_rsrc = make_rsrc(b_group, (uint32_t)p.N * (uint32_t)K);
        } else {
            sa_off = (uint32_t)(T.m0 + wave * 64 + lane) * 4u;
            b_rsrc = make_rsrc(p.b_q + (int64_t)T.g * p.N * K, (uint32_t)p.N * (uint32_t)K);
        }
        // B rows of DMA i are r0 + 8i; the swizzle of r0 + 8i only depends on i & 1
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int r = (wave * B_DMA + par) * 8 + (lane >> 3);
            b_off[par] = (uint32_t)(T.n0 + r) * (uint32_t)K + ((lane & 7) ^ swz(r)) * 16;  // rows past N read 0
        }
        // B scales of the tile's two 128-row blocks, all slices, into LDS by DMA
        // (no register round trip, so nothing here waits for them: they land
        // with slice 0).  Waves 0-3: block wave/2 (the second clamped when
        // N % 256 == 128), slices 64*(wave&1) + lane; lanes past the slice
        // count read past the end of the descriptor and write 0.
        if (!KG && wave < 4) {
            const int blk = min(T.n0 / 128 + (wave >> 1), nblk_per_g - 1);
            const int sl = (wave & 1) * 64 + lane;
            const auto bs_g = make_rsrc(p.b_s + (int64_t)T.g * nblk_per_g * ns, (uint32_t)(nblk_per_g * ns * 4));
            lds_dma4(bs_g, sl < ns ? (uint32_t)(blk * ns + sl) * 4u : 0x80000000u, 0u,
                     reinterpret_cast<char*>(g_bscale) + ((wave >> 1) * MAX_SLICES + (wave & 1) * 64) * 4);
        }
    };
    // DMA k (0 <= k < D) of one stage: A chunks, then B chunks, then the A scales
    auto issue_one = [&](auto stc, int slice, int k) {
        constexpr int ST = decltype(stc)::value;
        const bool live = slice < ns;
        const uint32_t koff = live ? (uint32_t)slice * BK : 0u;
        if (k < A_DMA) {
            lds_dma16(live ? a_rsrc : null_rsrc, a_off[k], koff, a_buf<ST, BM>() + (wave * A_DMA + k) * 1024);
        } else if (k < A_DMA + B_DMA) {
            const int i = k - A_DMA;
            lds_dma16<C::B_AUX>(live ? b_rsrc : null_rsrc, b_off[i & 1] + (uint32_t)((i & ~1) * 8) * (uint32_t)K, koff,
                      b_buf<ST>() + (wave * B_DMA + i) * 1024);
        } else if constexpr (KG) {
            lds_dma4(live ? (wave * 64 < BM ? sa_rsrc : wave * 64 == BM ? bs_rsrc : null_rsrc) : null_rsrc, sa_off,
                     live ? (uint32_t)slice * 4u : 0u, reinterpret_cast<char*>(sa_buf<ST>()) + wave * 256);
        } else {
            lds_dma4((live && wave * 64 < BM) ? sa_rsrc : null_rsrc, sa_off,
                     live ? (uint32_t)slice * p.sa_stride : 0u,
                     reinterpret_cast<char*>(sa_buf<ST>()) + wave * 256);
        }
    };
    auto issue = [&](auto stc, int slice) {
#pragma unroll
        for (int k = 0; k < D; ++k) issue_one(stc, slice, k);
    };

    int sbrow0, sbrow1;   // which of the two B blocks scales this wave's column tiles
    if constexpr (EPI == EPI_STORE_F32) {
        sbrow0 = (wn * WN_COLS) / 128;
        sbrow1 = sbrow0;
    } else {
        sbrow0 = 0;
        sbrow1 = 1;
    }
    // lane offsets of the fragment chunks; the wave's row/column base is folded in
    const uint32_t sw0 = (uint32_t)(((2 * kb) ^ swz(lr)) << 4);
    const uint32_t sw1 = (uint32_t)(((2 * kb + 1) ^ swz(lr)) << 4);
    const uint32_t a_lo0 = (uint32_t)(wm * WROWS + lr) * 128 + sw0;
    const uint32_t a_lo1 = (uint32_t)(wm * WROWS + lr) * 128 + sw1;
    const uint32_t bcol = (uint32_t)(ncol<EPI, C>(wn, 0) - ncol<EPI, C>(0, 0) + lr);
    const uint32_t b_lo0 = bcol * 128 + sw0;
    const uint32_t b_lo1 = bcol * 128 + sw1;
    const int sa_row = wm * WROWS + lr;      // this lane's output row inside the tile (+ mi * 16)

    v4f acc[MI][NI];

    // Ping-pong schedule.  The waves form two groups, waves 0-3 and 4-7, one
    // wave of each on every SIMD.  Every wave works a slice in two phases: a
    // memory phase (read the slice's A and B fragments and scales from LDS
    // into registers, issue the DMAs of slice s+2) and a matrix phase (the 16
    // MFMAs and the scale FMAs, registers only), with a workgroup barrier
    // before each phase.  Both groups run the same instruction stream, but
    // group 1 passes one extra barrier when a tile starts (and group 0 one
    // when it ends), so group 1 is one phase behind:
    //     phase 2s:   group 0 memory(s),  group 1 matrix(s-1)
    //     phase 2s+1: group 0 matrix(s),  group 1 memory(s)
    // and on each SIMD one wave feeds the matrix core while the other loads.
    // Stage reuse: the DMAs of slice s+2 (issued in phases 2s and 2s+1) go to
    // the stage of slice s-1, whose last reader (group 1, phase 2s-1) finished
    // before the barrier that opens phase 2s.  Data: the barrier that opens
    // phase 2s must see every wave's DMAs of slice s complete.  For group 0
    // it precedes memory(s), and its newer DMAs are those of slice s+1; for
    // group 1 it precedes matrix(s-1), and its newer DMAs are again those of
    // slice s+1: both wait for vmcnt(D).  The barrier before group 0's matrix
    // phase has no data to wait for (slices s+1 and s+2 may be in flight:
    // vmcnt(2D)).  The "memory" clobber keeps the compiler from moving LDS
    // accesses across a barrier, the scheduling barriers keep it from moving
    // MFMAs across.
#define MOE_STAGE_BARRIER(N) asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" ::: "memory")
    const bool lead = wave < NWAVES / 2;           // group 0
    auto barrier_mem = [&]() {                     // opens a memory phase
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (D == 7) MOE_STAGE_BARRIER(7);
        else MOE_STAGE_BARRIER(6);
        __builtin_amdgcn_sched_barrier(0);
    };
    // opens a matrix phase.  The wait count depends on the group; it is chosen
    // inside one asm block (every lane of a wave gives the same comparison, so
    // vcc is all ones or all zeros) so that the K loop has no branch the
    // compiler can see: a visible one costs registers and lets it move the
    // scale FMAs across barriers.
    auto barrier_mat = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (D == 7)
            asm volatile("v_cmp_gt_u32 vcc, %0, %1\n\ts_cbranch_vccz 1f\n\ts_waitcnt vmcnt(14)\n\ts_branch 2f\n"
                         "1:\n\ts_waitcnt vmcnt(7)\n2:\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                         :: "n"(NT / 2), "v"(tid) : "memory", "vcc");
        else
            asm volatile("v_cmp_gt_u32 vcc, %0, %1\n\ts_cbranch_vccz 1f\n\ts_waitcnt vmcnt(12)\n\ts_branch 2f\n"
                         "1:\n\ts_waitcnt vmcnt(6)\n2:\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                         :: "n"(NT / 2), "v"(tid) : "memory", "vcc");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto plain_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // The slice a wave is working on, as its memory phase left it.
    constexpr int NC = TR ? 1 : 4;
    v8i bfr[NI], afr[MI];
    float sav[MI][NC];
    float sb0 = 0.f, sb1 = 0.f;

    // Memory phase of slice s on stage ST.  A tile's first slice also issues
    // slice 1 (the tile prologue issues slice 0 only).
    auto mem_phase = [&](auto stc, int s, auto firstc) {
        constexpr int ST = decltype(stc)::value;
        constexpr bool FIRST = decltype(firstc)::value;
        const char* At = a_buf<ST, BM>();
        const char* Bt = b_buf<ST>();
        const float* SAt = sa_buf<ST>();
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bfr[ni] = frag(Bt, ncol<EPI, C>(0, ni) * 128, b_lo0, b_lo1);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            afr[mi] = frag(At, mi * 16 * 128, a_lo0, a_lo1);
            // scales: with B first a lane's four results share one row (lr) and
            // one scale; with A first they are rows 4*kb + j of one column
            if constexpr (TR) {
                sav[mi][0] = SAt[sa_row + mi * 16];
            } else {
                const float4 t = *reinterpret_cast<const float4*>(SAt + wm * WROWS + 4 * kb + mi * 16);
                sav[mi][0] = t.x; sav[mi][1] = t.y; sav[mi][2] = t.z; sav[mi][3] = t.w;
            }
        }
        if constexpr (KG) {
            sb0 = SAt[BM + sbrow0];
            sb1 = SAt[BM + sbrow1];
        } else {
            sb0 = g_bscale[sbrow0 * MAX_SLICES + s];
            sb1 = g_bscale[sbrow1 * MAX_SLICES + s];
        }
        if constexpr (FIRST && !EARLY1) issue(IC<(ST + 1) % NS>{}, s + 1);
        issue(IC<(ST + 2) % NS>{}, s + 2);
    };

    // Matrix phase: MFMA (mi, ni), then the four scale FMAs of (mi-1, ni),
    // whose partial finished four MFMAs earlier (the order is pinned by a
    // scheduling barrier after each MFMA).
    auto mat_phase = [&]() {
        auto fma4 = [&](const v4f& part, int mi, int ni, const float (&c0)[NC], const float (&c1)[NC]) {
            const bool second = (EPI != EPI_STORE_F32) && ni >= NI / 2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float c = second ? c1[TR ? 0 : j] : c0[TR ? 0 : j];
                acc[mi][ni][j] = __builtin_fmaf(part[j], c, acc[mi][ni][j]);
            }
        };
        v4f prev[NI];
        float p0[NC], p1[NC];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            float q0[NC], q1[NC];
            v4f cur[NI];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                if constexpr (TR)
                    cur[ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        bfr[ni], afr[mi], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                else
                    cur[ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        afr[mi], bfr[ni], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                if (mi > 0) fma4(prev[ni], mi - 1, ni, p0, p1);
                if (ni == NI - 1) {
#pragma unroll
                    for (int j = 0; j < NC; ++j) {
                        q0[j] = sav[mi][j] * sb0;
                        q1[j] = (EPI != EPI_STORE_F32) ? sav[mi][j] * sb1 : 0.f;
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) prev[ni] = cur[ni];
#pragma unroll
            for (int j = 0; j < NC; ++j) { p0[j] = q0[j]; p1[j] = q1[j]; }
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) fma4(prev[ni], MI - 1, ni, p0, p1);
    };

    // memory and matrix phase of a slice s >= 1 on stage ST
    auto slice_pair = [&](auto stc, int s) {
        barrier_mem();
        mem_phase(stc, s, std::false_type{});
        barrier_mat();
        mat_phase();
    };

    // FP32-store epilogue, through LDS: the tile's rows go 64 at a time into the
    // B buffers of stages 1 and 2 (32 rows of 1 KiB each; idle until the next
    // tile's second slice is issued), or for 32-row tiles into stage 2's alone
    // (stage 1 then takes the next tile's second slice during the
    // epilogue), then every wave writes whole rows, one
    // 16-byte piece per lane (128 store instructions per tile instead of 512
    // single floats).  In LDS the 16-float halves of each 32-float bank row
    // swap when bit 2 of the row is set: the four row groups of a fragment
    // write (A-first layout: lane holds rows 4*kb + j of column lr) then fall
    // on distinct banks, and a row read stays 1 KiB of whole 16-byte chunks.
    auto store_f32 = [&](const Tile& T) {
        if constexpr (EPI == EPI_STORE_F32) {
            constexpr int PASS_ROWS = BM < 64 ? BM : 64;
            constexpr int RPW = PASS_ROWS / NWAVES;            // rows each wave writes out per pass
            float* const buf0 = reinterpret_cast<float*>(BM == 32 ? g_b2 : g_b1);
            float* const buf1 = reinterpret_cast<float*>(g_b2);
            auto lds_at = [&](int lrow, int col) -> float* {      // lrow < PASS_ROWS
                float* b = lrow < 32 ? buf0 : buf1;
                return b + (lrow & 31) * 256 + (col ^ (((lrow >> 2) & 1) << 4));
            };
#pragma unroll
            for (int h = 0; h < BM / PASS_ROWS; ++h) {
                if ((wm * WROWS) / PASS_ROWS == h) {
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int lrow = wm * WROWS - h * PASS_ROWS + mi * 16 + kb * 4 + j;
#pragma unroll
                            for (int ni = 0; ni < NI; ++ni)
                                *lds_at(lrow, ncol<EPI, C>(wn, ni) + lr) = acc[mi][ni][j];
                        }
                }
                __syncthreads();
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const int lrow = wave * RPW + i;
                    const int r = h * PASS_ROWS + lrow;
                    const float* src = (lrow < 32 ? buf0 : buf1) + (lrow & 31) * 256 +
                                       4 * (lane ^ (((lrow >> 2) & 1) << 2));
                    const v4f v = *reinterpret_cast<const v4f*>(src);
                    const int n = T.n0 + 4 * lane;
                    if (r < T.rows && n < p.N) {
                        v4f* dst = reinterpret_cast<v4f*>(p.out + (int64_t)(T.m0 + r) * p.N + n);
                        // K-grouped tiles (a few slices each) are bound by this
                        // store: the non-temporal hint measured 4% faster there
                        if constexpr (KG) __builtin_nontemporal_store(v, dst);
                        else *dst = v;
                    }
                }
                if (h + 1 < BM / PASS_ROWS) __syncthreads();
            }
        }
    };

    // SwiGLU epilogues, in two parts around the next tile's first DMAs: the
    // arithmetic (scratch in stage 2, which the next tile's first two slices
    // leave alone), then the global stores.
    constexpr int HALF = NI / 2;
    constexpr int HC = WN_COLS / 2;          // h columns per wave
    float h[EPI == EPI_STORE_F32 ? 1 : MI][HALF > 0 ? HALF : 1][4];   // row sa_row + mi*16, h column wn*HC + ni*16 + 4*kb + j
    float* const amax_s = reinterpret_cast<float*>(g_b2);               // [WAVES_N][BM] row maxima
    float* const scale_s = amax_s + WAVES_N * BM;                        // [BM] row scales
    char* const qtile = a_buf<2, BM>();                                  // [BM][128] codes
    auto swiglu_compute = [&]() {
        if constexpr (EPI != EPI_STORE_F32) {
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < HALF; ++ni)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        h[mi][ni][j] = silu(acc[mi][ni][j]) * acc[mi][ni + HALF][j];
            if constexpr (EPI == EPI_SWIGLU_QUANT || EPI == EPI_SWIGLU_QUANT_Z) {
                // row maximum over this wave's HC h columns (lanes lr, lr+16, lr+32
                // and lr+48 hold one row), then across the N-waves in LDS
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    float m = 0.0f;
#pragma unroll
                    for (int ni = 0; ni < HALF; ++ni)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float a = __builtin_fabsf(h[mi][ni][j]);
                            m = a > m ? a : m;
                        }
#pragma unroll
                    for (int o = 16; o < 64; o <<= 1) {
                        const float other = __shfl_xor(m, o, 64);
                        m = other > m ? other : m;
                    }
                    if (kb == 0) amax_s[wn * BM + sa_row + mi * 16] = m;
                }
                __syncthreads();
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int r = sa_row + mi * 16;
                    float amax = amax_s[r];
#pragma unroll
                    for (int w = 1; w < WAVES_N; ++w) {
                        const float a = amax_s[w * BM + r];
                        amax = a > amax ? a : amax;
                    }
                    float inv, sc;
                    tile_scale(amax, inv, sc);
#pragma unroll
                    for (int ni = 0; ni < HALF; ++ni) {
                        const uint32_t w4 = e4m3_encode4(h[mi][ni][0] * inv, h[mi][ni][1] * inv,
                                                         h[mi][ni][2] * inv, h[mi][ni][3] * inv);
                        *reinterpret_cast<uint32_t*>(qtile + r * 128 + wn * HC + ni * 16 + 4 * kb) = w4;
                    }
                    if (wn == 0 && kb == 0) scale_s[r] = sc;
                }
                __syncthreads();
            }
        }
    };
    auto swiglu_store = [&](const Tile& T) {
        if constexpr (EPI != EPI_STORE_F32) {
            const int I = p.N / 2;
            const int h0 = T.n0 / 2;         // first h column of this tile
            if constexpr (EPI == EPI_SWIGLU_QUANT || EPI == EPI_SWIGLU_QUANT_Z) {
                // BM rows x 128 bytes, 16-byte stores, and one scale per row
                for (int c = tid; c < BM * 8; c += NT) {
                    const int r = c >> 3, part = c & 7;
                    if (r < T.rows)
                        *reinterpret_cast<uint4*>(p.out_q + (int64_t)(T.m0 + r) * I + h0 + part * 16) =
                            *reinterpret_cast<const uint4*>(qtile + r * 128 + part * 16);
                }
                if (tid < BM && tid < T.rows) p.out_s[(int64_t)(T.m0 + tid) * (I / 128) + h0 / 128] = scale_s[tid];
            }
            if (EPI == EPI_SWIGLU_F32 || (EPI == EPI_SWIGLU_QUANT && p.out)) {
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int r = sa_row + mi * 16;
                    if (r >= T.rows) continue;
                    float* orow = p.out + (int64_t)(T.m0 + r) * I + h0 + wn * HC + 4 * kb;
#pragma unroll
                    for (int ni = 0; ni < HALF; ++ni)
                        *reinterpret_cast<float4*>(orow + ni * 16) =
                            make_float4(h[mi][ni][0], h[mi][ni][1], h[mi][ni][2], h[mi][ni][3]);
                }
            }
            if constexpr (EPI == EPI_SWIGLU_QUANT_Z) {
                // the GEMM output z itself (gate and up columns in B's row order)
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int r = sa_row + mi * 16;
                    if (r >= T.rows) continue;
                    float* zrow = p.out + (int64_t)(T.m0 + r) * p.N + T.n0 + 4 * kb;
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni)
                        *reinterpret_cast<float4*>(zrow + ncol<EPI, C>(wn, ni)) =
                            make_float4(acc[mi][ni][0], acc[mi][ni][1], acc[mi][ni][2], acc[mi][ni][3]);
                }
            }
        }
    };

    // ---- the tile loop
    if (tid == 0) s_next = atomicAdd(p.counters + xcd, 1);
    __syncthreads();
    int t_cur = global_tile(__builtin_amdgcn_readfirstlane(s_next));
    if (t_cur < 0) return;
    Tile cur = tile_at(t_cur);
    load_rows(cur);
    setup(cur);
    issue(IC<0>{}, 0);
    if constexpr (EARLY1) issue(IC<1>{}, 1);
    // The tile after this one.  Its result is only needed after the K loop;
    // the library is built without the compiler's atomic optimizer, which
    // would otherwise consume it (and drain every DMA in flight) right here.
    int nxt_raw = 0;
    if (tid == 0) nxt_raw = atomicAdd(p.counters + xcd, 1);
    for (;;) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};
        // slice 0 landed (it and the previous tile's stores are all that is in
        // flight: a full wait); also publishes the B scales
        MOE_STAGE_BARRIER(0);
        __builtin_amdgcn_sched_barrier(0);

        if (!lead) plain_barrier();                // group 1: one phase behind
        mem_phase(IC<0>{}, 0, std::true_type{});
        barrier_mat();
        mat_phase();
        // whole rounds of three stages, then the remaining one or two slices
        int s = 1;
        for (; s + 3 <= ns; s += 3) {
            slice_pair(IC<1>{}, s);
            slice_pair(IC<2>{}, s + 1);
            slice_pair(IC<0>{}, s + 2);
        }
        if (s < ns) slice_pair(IC<1>{}, s);
        if (s + 1 < ns) slice_pair(IC<2>{}, s + 1);
        if (lead) plain_barrier();                 // group 0: catch up
        MOE_STAGE_BARRIER(0);      // drain the spare-stage DMAs before LDS is reused

        // next tile: its index was requested when this tile started
        if (tid == 0) s_next = nxt_raw;
        __syncthreads();
        const int t_nxt = global_tile(__builtin_amdgcn_readfirstlane(s_next));
        Tile nxt = cur;
        if (t_nxt >= 0) {
            nxt = tile_at(t_nxt);
            load_rows(nxt);
        }
        swiglu_compute();
        if (t_nxt >= 0) {
            setup(nxt);
            issue(IC<0>{}, 0);
            if constexpr (EARLY1) issue(IC<1>{}, 1);
            if (tid == 0) nxt_raw = atomicAdd(p.counters + xcd, 1);
        }
        store_f32(cur);
        swiglu_store(cur);
        if (t_nxt < 0) break;
        __syncthreads();   // stage-2 scratch and the tile's LDS reads are done before slice 2 lands
        cur = nxt;
    }
#undef MOE_STAGE_BARRIER
}

// ============================================================================
// The ring kernel: the tile computation above (non-K-grouped tiles), with one
// DMA ring that runs on across tiles.  Each block takes a static, XCD-aware
// share of the tile sequence (the same contiguous share per XCD as above, its
// tiles dealt round-robin to the XCD's blocks, so the 32 blocks of an XCD
// start and finish their tiles together and share A rows and B columns in
// the XCD's L2).  The next tile's first two slices are fetched during the
// last two slices of the current one, so a tile boundary costs no pipeline
// restart; the epilogues store straight from registers (the stores the
// barriers count are issued by every lane, and a lane without an output
// writes out of the buffer's range, which drops it), and the waits at the two
// barriers after an epilogue count those stores.  The next tile's record
// comes by one scalar load per tile; its gathered row indices and B-scale
// table reach LDS through the spare per-stage DMA slot, ahead of their use.
// Everything per tile is set up once per tile, so a slice's memory phase
// issues little beyond its DMAs and LDS reads (a SIMD issues a few scalar
// instructions per cycle at most, and the memory phase must stay shorter than
// the other wave's matrix phase).
//
// The three stages are one LDS object addressed at run time (a tile may start
// on any stage), so the DMAs are issued from inline asm: the compiler adds no
// waits of its own for them, and every wait is the explicit one in a barrier.
// Null DMAs (out-of-range offsets) still write zeros to their LDS slots; each
// one targets a slot nothing reads at that time.
// ============================================================================
constexpr int RING_MIN_SLICES = 4;           // the next tile's rows are fetched 4 slices ahead
constexpr int RING_SA_BYTES = 64 * NWAVES * 4;
constexpr int RING_A = 0, RING_B = A_MAX_BYTES, RING_SA = A_MAX_BYTES + B_BYTES;
constexpr int RING_STAGE = A_MAX_BYTES + B_BYTES + RING_SA_BYTES;   // 50 KiB
static_assert(RING_STAGE % 1024 == 0, "stage bases keep the swizzle's 1 KiB alignment");
__shared__ __attribute__((aligned(1024))) char g_ring[3 * RING_STAGE];
__shared__ __attribute__((aligned(16))) float g_btab[2][2 * MAX_SLICES];   // B scales of a tile, by tile parity
__shared__ __attribute__((aligned(16))) int32_t g_rowbuf[128];             // the next tile's gathered A rows
__shared__ __attribute__((aligned(16))) float g_rmax[512];                 // [WAVES_N][BM] row maxima of h

// Ring tile shape: 128 rows, 2 x 4 waves of 64 x 64 (one row group per half
// of the workgroup, so the SwiGLU row maxima are exchanged inside one
// ping-pong group).  Every epilogue puts B first in the MFMA: a lane's four
// results are four consecutive columns of one row, stored as one 16-byte (or
// 4-code) piece.
template <int BM_>
struct RCfg {
    static_assert(BM_ == 128, "the ring kernel runs 128-row tiles");
    static constexpr int BM = BM_;
    static constexpr int WAVES_M = 2, WAVES_N = 4;
    static constexpr int WROWS = BM_ / 2;
    static constexpr int MI = WROWS / 16;
    static constexpr int WN_COLS = BN / WAVES_N;           // 64
    static constexpr int NI = WN_COLS / 16;                // 4
    static constexpr int A_INSTR = BM_ * BK / 1024;
    static constexpr int A_COPIES = A_INSTR >= NWAVES ? 1 : NWAVES / A_INSTR;
    static constexpr int A_DMA = A_INSTR * A_COPIES / NWAVES;
    static constexpr int B_DMA = B_BYTES / 1024 / NWAVES;
    static constexpr int D = A_DMA + B_DMA + 1;            // + the per-wave dword slot
};

typedef int ring_v4i __attribute__((ext_vector_type(4)));
typedef unsigned ring_v4u __attribute__((ext_vector_type(4)));

// buffer descriptor in SGPRs (stride 0, byte-granular range check)
__device__ __forceinline__ ring_v4i ring_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    ring_v4i r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xFFFFu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}
// the value of lane 0 in an SGPR: inline asm's "s" operands must be wave-uniform
// values the compiler can see as such
__device__ __forceinline__ uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ ring_v4i uni(ring_v4i r) {
    ring_v4i o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __builtin_amdgcn_readfirstlane(r[i]);
    return o;
}
// global -> LDS DMA: lane l's bytes land at lds + l * size (lds wave-uniform).
// The LDS address goes through m0, set in the same asm block as the DMA that
// reads it.  The compiler warns that a clobbered m0 may not be preserved; the
// ring kernel's code has no other m0 user (its assembly writes m0 only in
// these blocks), so nothing live is lost.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void ring_dma16(ring_v4i r_, uint32_t voff, uint32_t soff_, uint32_t lds_) {
    const ring_v4i r = uni(r_);
    const uint32_t soff = uni(soff_), lds = uni(lds_);
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void ring_dma4(ring_v4i r_, uint32_t voff, uint32_t soff_, uint32_t lds_) {
    const ring_v4i r = uni(r_);
    const uint32_t soff = uni(soff_), lds = uni(lds_);
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
                 :: "v"(voff), "s"(r), "s"(soff), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

template <int EPI, int BM_>
__global__ __launch_bounds__(NT) void grouped_gemm_ring_kernel(GemmArgs p) {
    using C = RCfg<BM_>;
    constexpr int BM = C::BM, MI = C::MI, NI = C::NI, WAVES_N = C::WAVES_N;
    constexpr int WN_COLS = C::WN_COLS, WROWS = C::WROWS, A_DMA = C::A_DMA, B_DMA = C::B_DMA;
    constexpr int D = C::D;
    constexpr int HALF = NI / 2;
    constexpr int HC = WN_COLS / 2;                        // h columns per wave (SwiGLU)
    constexpr bool QUANT = (EPI == EPI_SWIGLU_QUANT || EPI == EPI_SWIGLU_QUANT_Z);
    // stores every wave issues per tile, unconditionally (see the epilogue).
    // A wave may issue more (the row scales from the waves of the first
    // column group, FP32 h when requested): more stores than counted only
    // make the waits below stricter, never looser.
    constexpr int S = EPI == EPI_STORE_F32 ? MI * NI
                    : EPI == EPI_SWIGLU_QUANT_Z ? MI * HALF + MI * NI
                    : MI * HALF;
    static_assert(D + S <= 63, "vmcnt holds 6 bits");
    static_assert(BM * WAVES_N <= 512, "row-maximum buffer");
    const int K = p.K, ns = K / BK;                        // ns >= RING_MIN_SLICES (host-checked)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int kb = lane >> 4;
    const int lr = lane & 15;
    const bool lead = wave < NWAVES / 2;

    // ---- static schedule: XCD x owns tiles [x*share, (x+1)*share) of the
    // sequence; its blocks take every nbx-th of them
    const int n_tiles = (p.N + BN - 1) / BN;
    const int total = __builtin_amdgcn_readfirstlane(p.tile_start[p.G]) * n_tiles;
    const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3, nbx = gridDim.x >> 3;
    const int share = (total + 7) >> 3;
    const int t_first = xcd * share + jx;
    const int t_end = min(total, xcd * share + share);
    if (t_first >= t_end) return;
    auto tile_no = [&](int k) {            // the k-th tile of this block, -1 past its share
        const int t = t_first + k * nbx;
        return t < t_end ? t : -1;
    };

    struct Tile { int g, m0, rows, n0; };
    const int m_total = (int)(p.sa_stride / 4u);
    // a record with every field clamped into range: whatever a record holds,
    // the DMA and store descriptors built from it stay inside their buffers
    auto clamp_tile = [&](int g, int m0, int rows, int n0) {
        Tile T;
        T.g = __builtin_amdgcn_readfirstlane(min(max(g, 0), p.G - 1));
        T.m0 = __builtin_amdgcn_readfirstlane(min(max(m0, 0), m_total - 1));
        T.rows = __builtin_amdgcn_readfirstlane(min(max(rows, 1), min(BM, m_total - T.m0)));
        T.n0 = __builtin_amdgcn_readfirstlane(min(max(n0, 0), p.N - 1));
        return T;
    };
    // the record of tile t, by one scalar load (waited for in the same asm block)
    auto load_tile = [&](int t) {
        const int4* ptr = p.tiles + t;
        int4 v;
        asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
        return clamp_tile(v.x, v.y, v.z, v.w);
    };

    // ---- descriptors and LDS addresses (wave-uniform)
    const ring_v4i a_rsrc = ring_rsrc(p.a_q, 0xFFFFFFFFu);
    const ring_v4i sa_rsrc = ring_rsrc(p.a_sT, p.sa_stride * (uint32_t)ns);   // rows past M_total read 0
    const int nblk = p.N / 128;
    const uint32_t ring0 = lds_addr(g_ring);
    const uint32_t ring_last = ring0 + 2 * RING_STAGE;
    constexpr uint32_t OOR = 0x80000000u;  // an offset past every descriptor's range
    // the per-stage dword slot of each wave: A scales (waves below BM/64,
    // every slice), the next tile's B-scale table (waves 2-5, at its slice
    // ns-2), the next tile's gathered rows (waves 6-7, at slice ns-4), or
    // nothing: an inactive slot DMAs out of range into the wave's unused
    // scale slot of the stage being written
    const bool x_ascale = wave * 64 < BM;
    const bool x_btab = !x_ascale && wave >= 2 && wave <= 5;
    const bool x_rows = !x_ascale && wave >= 6 && p.a_rows != nullptr;
    const ring_v4i x_rsrc = uni(x_ascale ? sa_rsrc
                                : x_btab ? ring_rsrc(p.b_s, (uint32_t)p.G * (uint32_t)nblk * (uint32_t)ns * 4u)
                                : ring_rsrc(p.a_rows ? (const void*)p.a_rows : (const void*)p.a_q,
                                            p.a_rows ? p.sa_stride : 0u));
    uint32_t x_voff = OOR, x_dst = 0;
    int x_phase = -1;                      // the slice whose memory phase issues this wave's slot DMA
    // slot parameters for the next tile nx (par: its B-table buffer)
    auto set_slot = [&](const Tile& nx, bool has_nx, int par) {
        x_phase = -1;
        if (x_btab) {
            const int q = wave - 2;
            const int blk = min(nx.n0 / 128 + (q >> 1), nblk - 1), sl = (q & 1) * 64 + lane;
            x_voff = sl < ns ? (uint32_t)((nx.g * nblk + blk) * ns + sl) * 4u : OOR;
            x_dst = lds_addr(&g_btab[par][(q >> 1) * MAX_SLICES + (q & 1) * 64]);
            x_phase = has_nx ? ns - 2 : -1;
        } else if (x_rows) {
            const int r = (wave - 6) * 64 + lane;
            x_voff = r < BM ? (uint32_t)(nx.m0 + r) * 4u : OOR;
            x_dst = lds_addr(&g_rowbuf[(wave - 6) * 64]);
            x_phase = has_nx ? ns - 4 : -1;
        }
        x_phase = __builtin_amdgcn_readfirstlane(x_phase);
        x_dst = uni(x_dst);
    };

    // ---- the fetch cursor: the tile whose slices the DMAs read (the current
    // one, then from its slice ns-2 on the next), its per-lane sources, and
    // the slice issued next
    uint32_t fa_off[A_DMA], fb_off[2], f_sa_off;
    ring_v4i fb_rsrc;
    int fslice;
    auto set_fetch = [&](const Tile& T, bool rows_in_lds) {
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int r = ((wave * A_DMA + i) % C::A_INSTR) * 8 + (lane >> 3);
            const int rr = min(r, T.rows - 1);
            uint32_t am;
            if (!p.a_rows) am = (uint32_t)(T.m0 + rr);
            else if (rows_in_lds) am = (uint32_t)g_rowbuf[rr];   // indices of rows of a_q, or 0
            else am = (uint32_t)p.a_rows[T.m0 + rr];
            fa_off[i] = am * (uint32_t)K + ((lane & 7) ^ swz(r)) * 16;
        }
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            const int r = (wave * B_DMA + par) * 8 + (lane >> 3);
            fb_off[par] = (uint32_t)(T.n0 + r) * (uint32_t)K + ((lane & 7) ^ swz(r)) * 16;   // rows past N read 0
        }
        f_sa_off = (uint32_t)(T.m0 + wave * 64 + lane) * 4u;
        fb_rsrc = uni(ring_rsrc(p.b_q + (int64_t)T.g * p.N * K, (uint32_t)p.N * (uint32_t)K));
    };
    // the DMAs of the cursor's slice into the stage at LDS address dst
    auto issue = [&](uint32_t dst) {
        const uint32_t koff = uni((uint32_t)fslice * BK);
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) ring_dma16(a_rsrc, fa_off[i], koff, dst + RING_A + (wave * A_DMA + i) * 1024);
#pragma unroll
        for (int i = 0; i < B_DMA; ++i)
            ring_dma16(fb_rsrc, fb_off[i & 1] + (uint32_t)((i & ~1) * 8) * (uint32_t)K, koff,
                                 dst + RING_B + (wave * B_DMA + i) * 1024);
    };
    auto issue_slot = [&](uint32_t dst, int s) {
        if (x_ascale) {
            ring_dma4(x_rsrc, f_sa_off, uni((uint32_t)fslice * p.sa_stride), dst + RING_SA + wave * 256);
        } else {
            const bool on = s == x_phase;
            ring_dma4(x_rsrc, on ? x_voff : OOR, 0u, uni(on ? x_dst : dst + RING_SA + wave * 256));
        }
    };

    // ---- fragment offsets (as in grouped_gemm_kernel; B first)
    const uint32_t sw0 = (uint32_t)(((2 * kb) ^ swz(lr)) << 4);
    const uint32_t sw1 = (uint32_t)(((2 * kb + 1) ^ swz(lr)) << 4);
    const uint32_t a_lo0 = (uint32_t)(wm * WROWS + lr) * 128 + sw0;
    const uint32_t a_lo1 = (uint32_t)(wm * WROWS + lr) * 128 + sw1;
    const uint32_t bcol = (uint32_t)(ncol<EPI, C>(wn, 0) - ncol<EPI, C>(0, 0) + lr);
    const uint32_t b_lo0 = bcol * 128 + sw0;
    const uint32_t b_lo1 = bcol * 128 + sw1;
    const int sa_row = wm * WROWS + lr;
    int sbrow0, sbrow1;
    if constexpr (EPI == EPI_STORE_F32) {
        sbrow0 = (wn * WN_COLS) / 128;
        sbrow1 = sbrow0;
    } else {
        sbrow0 = 0;
        sbrow1 = 1;
    }

    v4f acc[MI][NI];
    v8i bfr[NI], afr[MI];
    float sav[MI];
    float sb0 = 0.f, sb1 = 0.f;
    auto mem_reads = [&](const char* stage, int s, int par) {
        const char* At = stage + RING_A;
        const char* Bt = stage + RING_B;
        const float* SAt = reinterpret_cast<const float*>(stage + RING_SA);
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) bfr[ni] = frag(Bt, ncol<EPI, C>(0, ni) * 128, b_lo0, b_lo1);
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            afr[mi] = frag(At, mi * 16 * 128, a_lo0, a_lo1);
            sav[mi] = SAt[sa_row + mi * 16];
        }
        sb0 = g_btab[par][sbrow0 * MAX_SLICES + s];
        sb1 = g_btab[par][sbrow1 * MAX_SLICES + s];
    };
    // MFMA (mi, ni) into a fresh accumulator, then the four scale FMAs of
    // (mi-1, ni), whose partial finished four MFMAs earlier
    auto mat_phase = [&]() {
        auto fma4 = [&](const v4f& part, int mi, int ni, float c0, float c1) {
            const float c = ((EPI != EPI_STORE_F32) && ni >= HALF) ? c1 : c0;
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mi][ni][j] = __builtin_fmaf(part[j], c, acc[mi][ni][j]);
        };
        v4f prev[NI];
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
            float q0 = 0.f, q1 = 0.f;
            v4f cur[NI];
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
                cur[ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    bfr[ni], afr[mi], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                if (mi > 0) fma4(prev[ni], mi - 1, ni, p0, p1);
                if (ni == NI - 1) {
                    q0 = sav[mi] * sb0;
                    q1 = (EPI != EPI_STORE_F32) ? sav[mi] * sb1 : 0.f;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) prev[ni] = cur[ni];
            p0 = q0;
            p1 = q1;
        }
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) fma4(prev[ni], MI - 1, ni, p0, p1);
    };

    // ---- barriers.  Group 1 (waves 4-7) runs one barrier behind group 0, so
    // each hardware barrier is one group's "memory" barrier and the other's
    // "matrix" barrier; the waits below follow from each wave's own stream of
    // vector-memory ops (D DMAs per memory phase, S stores per epilogue).
    //   barrier_mem (before reading slice s): slice s landed; the most recent
    //     ops are the D DMAs of slice s+1, plus, for the first two slices
    //     after an epilogue (pend > 0), that epilogue's S stores: vmcnt(D) or
    //     vmcnt(D + S).
    //   barrier_mat: group 0 needs nothing (group 1 then reads a slice that
    //     the previous barrier saw land); group 1's coincides with group 0's
    //     next memory barrier, so it waits for slice s+1: vmcnt(D), or
    //     vmcnt(D + S) at the first slice after an epilogue (pend == 2), or
    //     nothing at the last slice of a SwiGLU-quant tile (the row-maximum
    //     barrier that follows takes that wait).
    auto barrier_mem = [&](int pend) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_cmp_eq_u32 %0, 0\n\ts_cbranch_scc1 1f\n\ts_waitcnt vmcnt(%1)\n\ts_branch 2f\n"
                     "1:\n\ts_waitcnt vmcnt(%2)\n2:\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                     :: "s"(pend), "n"(D + S), "n"(D) : "memory", "scc");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto barrier_sel = [&](int sel) {      // 0: no vector-memory wait, 1: vmcnt(D + S), 2: vmcnt(D)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_cmp_eq_u32 %0, 2\n\ts_cbranch_scc1 3f\n\ts_cmp_eq_u32 %0, 1\n\ts_cbranch_scc1 4f\n"
                     "\ts_branch 5f\n3:\n\ts_waitcnt vmcnt(%1)\n\ts_branch 5f\n4:\n\ts_waitcnt vmcnt(%2)\n"
                     "5:\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier"
                     :: "s"(sel), "n"(D), "n"(D + S) : "memory", "scc");
        __builtin_amdgcn_sched_barrier(0);
    };
    auto plain_barrier = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_barrier" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- epilogues: the S counted stores are issued by every lane of every
    // wave; a lane without an output (row past the tile, column past N) gets
    // an offset past its buffer's range, so the hardware drops it.
    auto store_b128 = [&](const v4f& v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(ring_v4u, v), r, (int)off, 0, 0);
    };
    // off if ok, else an offset past any range below 2^31 (every output
    // descriptor here covers less): bitwise, so no lane-dependent branch
    // splits a store in two
    auto keep = [](uint32_t off, bool ok) -> uint32_t { return off | (OOR & (0u - (uint32_t)!ok)); };
    auto epilogue = [&](const Tile& T) {
        const int I = p.N / 2;
        const int h0 = T.n0 / 2;
        if constexpr (EPI == EPI_STORE_F32) {
            const auto orsrc = make_rsrc(p.out + (int64_t)T.m0 * p.N, (uint32_t)T.rows * (uint32_t)p.N * 4u);
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < NI; ++ni) {
                    const int r = wm * WROWS + mi * 16 + lr;
                    const int c = T.n0 + ncol<EPI, C>(wn, ni) + 4 * kb;
                    store_b128(acc[mi][ni], orsrc,
                               keep(((uint32_t)r * (uint32_t)p.N + (uint32_t)c) * 4u, (r < T.rows) & (c < p.N)));
                }
        } else {
            float h[MI][HALF][4];
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < HALF; ++ni)
#pragma unroll
                    for (int j = 0; j < 4; ++j) h[mi][ni][j] = silu(acc[mi][ni][j]) * acc[mi][ni + HALF][j];
            // h columns h0 + wn*HC + ni*16 + 4*kb .. +3 of row m0 + r
            auto h_off = [&](int r, int ni, uint32_t elem) -> uint32_t {
                return keep(((uint32_t)r * (uint32_t)I + (uint32_t)(h0 + wn * HC + ni * 16 + 4 * kb)) * elem, r < T.rows);
            };
            if (EPI == EPI_SWIGLU_F32 || (EPI == EPI_SWIGLU_QUANT && p.out)) {
                // FP32 h (required for SWIGLU_F32, optional for SWIGLU_QUANT;
                // counted in S only for SWIGLU_F32)
                const auto hrsrc = make_rsrc(p.out + (int64_t)T.m0 * I, (uint32_t)T.rows * (uint32_t)I * 4u);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < HALF; ++ni)
                        store_b128(v4f{h[mi][ni][0], h[mi][ni][1], h[mi][ni][2], h[mi][ni][3]}, hrsrc,
                                   h_off(wm * WROWS + mi * 16 + lr, ni, 4u));
            }
            if constexpr (QUANT) {
                // row maxima over the tile's 128 h columns: lanes lr, lr+16,
                // lr+32, lr+48 hold one row; then across the N-waves of the
                // row group through LDS
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    float m = 0.0f;
#pragma unroll
                    for (int ni = 0; ni < HALF; ++ni)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const float a = __builtin_fabsf(h[mi][ni][j]);
                            m = a > m ? a : m;
                        }
#pragma unroll
                    for (int o = 16; o < 64; o <<= 1) {
                        const float other = __shfl_xor(m, o, 64);
                        m = other > m ? other : m;
                    }
                    if (kb == 0) g_rmax[wn * BM + wm * WROWS + mi * 16 + lr] = m;
                }
                barrier_sel(lead ? 0 : 2);      // group 1: the next tile's slice 0 (group 0 reads it next)
                const auto qrsrc = make_rsrc(p.out_q + (int64_t)T.m0 * I, (uint32_t)T.rows * (uint32_t)I);
                const auto srsrc = make_rsrc(p.out_s + (int64_t)T.m0 * (I / 128), (uint32_t)T.rows * (uint32_t)(I / 128) * 4u);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi) {
                    const int r = wm * WROWS + mi * 16 + lr;
                    float amax = g_rmax[wm * WROWS + mi * 16 + lr];
#pragma unroll
                    for (int w = 1; w < WAVES_N; ++w) {
                        const float a = g_rmax[w * BM + wm * WROWS + mi * 16 + lr];
                        amax = a > amax ? a : amax;
                    }
                    float inv, sc;
                    tile_scale(amax, inv, sc);
#pragma unroll
                    for (int ni = 0; ni < HALF; ++ni) {
                        const uint32_t w4 = e4m3_encode4(h[mi][ni][0] * inv, h[mi][ni][1] * inv,
                                                         h[mi][ni][2] * inv, h[mi][ni][3] * inv);
                        __builtin_amdgcn_raw_buffer_store_b32(w4, qrsrc, (int)h_off(r, ni, 1u), 0, 0);
                    }
                    if (wn == 0) {                 // one scale per row, from the first column group
                        const uint32_t soff = keep(((uint32_t)r * (uint32_t)(I / 128) + (uint32_t)(h0 / 128)) * 4u,
                                                   (kb == 0) & (r < T.rows));
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sc), srsrc, (int)soff, 0, 0);
                    }
                }
            }
            if constexpr (EPI == EPI_SWIGLU_QUANT_Z) {
                // the GEMM output z itself (gate and up columns in B's row order)
                const auto zrsrc = make_rsrc(p.out + (int64_t)T.m0 * p.N, (uint32_t)T.rows * (uint32_t)p.N * 4u);
#pragma unroll
                for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                    for (int ni = 0; ni < NI; ++ni) {
                        const int r = wm * WROWS + mi * 16 + lr;
                        store_b128(acc[mi][ni], zrsrc,
                                   keep(((uint32_t)r * (uint32_t)p.N + (uint32_t)(T.n0 + ncol<EPI, C>(wn, ni) + 4 * kb)) * 4u,
                                        r < T.rows));
                    }
            }
        }
    };

    // ---- prologue: tile 0's record, rows and B scales read directly, slices
    // 0 and 1 of tile 0 issued, the next tile's record loaded; everything
    // drained before the ping-pong starts
    int k = 0;
    Tile cur = load_tile(t_first);
    int t_nx = tile_no(1);
    Tile nx = cur;
    if (t_nx >= 0) nx = load_tile(t_nx);
    for (int i = tid; i < 2 * MAX_SLICES; i += NT) {
        const int blk = min(cur.n0 / 128 + i / MAX_SLICES, nblk - 1), sl = i % MAX_SLICES;
        g_btab[0][i] = sl < ns ? p.b_s[((int64_t)cur.g * nblk + blk) * ns + sl] : 0.0f;
    }
    set_fetch(cur, false);
    for (fslice = 0; fslice < 2; ++fslice) {
        const uint32_t dst = ring0 + (uint32_t)fslice * RING_STAGE;
        issue(dst);
        issue_slot(dst, -2);               // A scales; every other slot is inactive here
    }
    set_slot(nx, t_nx >= 0, 1);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (!lead) plain_barrier();            // group 1: one barrier behind from here on

    uint32_t rd = ring0, wr = ring_last;   // LDS stages read and written by the current memory phase
    int pend = 0;                          // slices left whose waits must count an epilogue's stores
    for (;;) {
        const bool has_nx = t_nx >= 0;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < ns; ++s) {
            barrier_mem(pend);
            mem_reads(g_ring + (rd - ring0), s, k & 1);
            if (s == ns - 2) {
                // the cursor moves to the next tile (its gathered rows landed
                // with slice ns-2); past the last tile it re-reads this tile's
                // first slices into stages nothing reads again
                if (has_nx) set_fetch(nx, true);
                fslice = 0;
            }
            issue(wr);
            issue_slot(wr, s);
            ++fslice;
            barrier_sel(lead ? 0 : pend == 2 ? 1 : (QUANT && s == ns - 1) ? 0 : 2);
            mat_phase();
            rd = rd == ring_last ? ring0 : rd + RING_STAGE;
            wr = wr == ring_last ? ring0 : wr + RING_STAGE;
            pend = pend > 0 ? pend - 1 : 0;
        }
        epilogue(cur);
        if (!has_nx) break;
        ++k;
        cur = nx;
        t_nx = tile_no(k + 1);
        if (t_nx >= 0) nx = load_tile(t_nx);
        set_slot(nx, t_nx >= 0, (k + 1) & 1);
        pend = 2;
    }
    if (lead) plain_barrier();             // group 0: catch up
    // every DMA lands before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
}

// tile_start[g] = sum_{g' < g} ceil(rows_g' / BM), for g = 0..G; zeroes the
// 8 per-XCD tile counters that follow it.
__global__ __launch_bounds__(256) void gemm_tile_map_kernel(const int32_t* __restrict__ go,
                                                            int G, int BM, int32_t* __restrict__ ts) {
    if (threadIdx.x < 8) ts[G + 1 + threadIdx.x] = 0;
    __shared__ int32_t buf[256];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < G; base += 256) {
        const int g = base + threadIdx.x;
        const int32_t v = (g < G) ? (go[g + 1] - go[g] + BM - 1) / BM : 0;
        buf[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int32_t x = (threadIdx.x >= (unsigned)off) ? buf[threadIdx.x - off] : 0;
            __syncthreads();
            buf[threadIdx.x] += x;
            __syncthreads();
        }
        if (g < G) ts[g] = carry + buf[threadIdx.x] - v;
        __syncthreads();
        if (threadIdx.x == 255) carry += buf[255];
        __syncthreads();
    }
    if (threadIdx.x == 0) ts[G] = carry;
}

// The tile sequence: tile t = (row tile q, column tile) with q = t / n_tiles in
// group g (tile_start[g] <= q < tile_start[g+1]); inside a group, chunks of
// up to GROUP_M row tiles, the column tile slow inside a chunk.
__global__ __launch_bounds__(256) void gemm_tile_list_kernel(const int32_t* __restrict__ go,
                                                             const int32_t* __restrict__ ts, int G,
                                                             int BM, int N, int4* __restrict__ tiles) {
    const int n_tiles = (N + BN - 1) / BN;
    const int total = ts[G] * n_tiles;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    const int q = t / n_tiles;
    int lo = 0, hi = G - 1;                       // largest g with ts[g] <= q
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (ts[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int mt_g = ts[lo + 1] - ts[lo];
    const int local = t - ts[lo] * n_tiles;
    const int chunk = local / (GROUP_M * n_tiles);
    const int chunk_rows = min(GROUP_M, mt_g - chunk * GROUP_M);
    const int in_chunk = local - chunk * GROUP_M * n_tiles;
    const int m0 = go[lo] + (chunk * GROUP_M + in_chunk % chunk_rows) * BM;
    tiles[t] = make_int4(lo, m0, min(BM, go[lo + 1] - m0), (in_chunk / chunk_rows) * BN);
}

// a_sT[j][m] = a_s[am][j] with am = a_rows[m] (or m): the A scales gathered
// into GEMM row order and made slice-major, so that the scales of one slice
// for a tile's rows are contiguous.  One block per 64 rows, through LDS.
// The slice-major copy of the A scales of rows m0 .. m0+63 (one 256-thread
// block): four threads per row take the row's source index once and read its
// ns scales (thread q of the row reads slices q, q+4, ...; all its loads go
// out before its first LDS store), then the block writes each slice's 64
// consecutive rows.
__device__ __forceinline__ void gather_scales_64(const float* __restrict__ a_s, const int32_t* __restrict__ a_rows,
                                                 int64_t M_total, int ns, float* __restrict__ a_sT, int64_t m0,
                                                 float (*t)[MAX_SLICES + 1]) {
    constexpr int PER_Q = MAX_SLICES / 4;
    const int tid = threadIdx.x;
    const int r = tid >> 2, qq = tid & 3;
    const int64_t m = m0 + r;
    const bool live = m < M_total;
    const float* row = a_s + (live ? (a_rows ? (int64_t)a_rows[m] : m) : 0) * ns;
    float v[PER_Q];
#pragma unroll
    for (int k = 0; k < PER_Q; ++k) {
        const int j = qq + 4 * k;
        v[k] = (live && j < ns) ? row[j] : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < PER_Q; ++k) {
        const int j = qq + 4 * k;
        if (j < ns) t[r][j] = v[k];
    }
    __syncthreads();
    for (int i = tid; i < 64 * ns; i += 256) {
        const int j = i >> 6, rr = i & 63;
        const int64_t mm = m0 + rr;
        if (mm < M_total) a_sT[j * M_total + mm] = t[rr][j];
    }
}

__global__ __launch_bounds__(256) void gemm_scale_gather_kernel(const float* __restrict__ a_s,
                                                                const int32_t* __restrict__ a_rows,
                                                                int64_t M_total, int ns,
                                                                float* __restrict__ a_sT) {
    __shared__ float t[64][MAX_SLICES + 1];
    gather_scales_64(a_s, a_rows, M_total, ns, a_sT, (int64_t)blockIdx.x * 64, t);
}

// The three preparation steps above in one launch, for G <= PREP_MAX_G (the
// kernels are short, and each launch of its own costs several microseconds):
// blocks [0, nl) build the tile list, each from its own LDS copy of the tile
// starts (block 0 also writes them to the workspace and zeroes the per-XCD
// counters); blocks [nl, nl + ceil(M_total / 64)) gather the A scales.
constexpr int PREP_MAX_G = 4096;

__global__ __launch_bounds__(256) void gemm_prep_kernel(const int32_t* __restrict__ go, int G, int BM,
                                                        int N, int nl, int32_t* __restrict__ ts,
                                                        int4* __restrict__ tiles,
                                                        const float* __restrict__ a_s,
                                                        const int32_t* __restrict__ a_rows,
                                                        int64_t M_total, int ns,
                                                        float* __restrict__ a_sT) {
    __shared__ int32_t lts[PREP_MAX_G + 1];
    __shared__ int32_t part[256];
    __shared__ float t[64][MAX_SLICES + 1];
    if ((int)blockIdx.x >= nl) {
        gather_scales_64(a_s, a_rows, M_total, ns, a_sT, (int64_t)(blockIdx.x - nl) * 64, t);
        return;
    }
    // exclusive scan of ceil(rows_g / BM): thread i owns groups [i*c, i*c + c)
    const int c = (G + 255) / 256;
    const int g0 = threadIdx.x * c;
    int32_t sum = 0;
    for (int g = g0; g < g0 + c && g < G; ++g) sum += (go[g + 1] - go[g] + BM - 1) / BM;
    part[threadIdx.x] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
        const int32_t x = (threadIdx.x >= (unsigned)off) ? part[threadIdx.x - off] : 0;
        __syncthreads();
        part[threadIdx.x] += x;
        __syncthreads();
    }
    int32_t run = part[threadIdx.x] - sum;
    for (int g = g0; g < g0 + c && g < G; ++g) {
        lts[g] = run;
        run += (go[g + 1] - go[g] + BM - 1) / BM;
    }
    if (threadIdx.x == 255) lts[G] = part[255];
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int g = threadIdx.x; g <= G; g += 256) ts[g] = lts[g];
        if (threadIdx.x < 8) ts[G + 1 + threadIdx.x] = 0;
    }
    // this block's part of the tile list (as gemm_tile_list_kernel)
    const int n_tiles = (N + BN - 1) / BN;
    const int total = lts[G] * n_tiles;
    const int tt = blockIdx.x * 256 + threadIdx.x;
    if (tt >= total) return;
    const int q = tt / n_tiles;
    int lo = 0, hi = G - 1;                       // largest g with lts[g] <= q
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (lts[mid] <= q) lo = mid; else hi = mid - 1;
    }
    const int mt_g = lts[lo + 1] - lts[lo];
    const int local = tt - lts[lo] * n_tiles;
    const int chunk = local / (GROUP_M * n_tiles);
    const int chunk_rows = min(GROUP_M, mt_g - chunk * GROUP_M);
    const int in_chunk = local - chunk * GROUP_M * n_tiles;
    const int m0 = go[lo] + (chunk * GROUP_M + in_chunk % chunk_rows) * BM;
    tiles[tt] = make_int4(lo, m0, min(BM, go[lo + 1] - m0), (in_chunk / chunk_rows) * BN);
}

// CU count of the calling thread's current device, cached per device (any
// thread may call; a lost race only repeats the query)
int cu_count_for_current_device() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        c = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
                ? n : 256;
        cached[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

}  // namespace

// [tile_start: G+1][counters: 8] (16-byte aligned) [tile list: int4 per tile, bound for
// 32-row tiles] (256-byte aligned) [A scales, slice-major: K/128 x M_total FP32]
static int64_t tile_list_offset(int G) { return ((int64_t)(G + 1 + 8) * 4 + 15) / 16 * 16; }
static int64_t tile_bound(int G, int64_t M_total, int N) {
    return ((M_total + 31) / 32 + G) * (int64_t)((N + BN - 1) / BN);
}
static int64_t scale_copy_offset(int G, int64_t M_total, int N) {
    return (tile_list_offset(G) + tile_bound(G, M_total, N) * 16 + 255) / 256 * 256;
}

size_t gemm_ws_bytes(int G, int64_t M_total, int N, int K) {
    return (size_t)(scale_copy_offset(G, M_total, N) + (int64_t)(K / BK) * M_total * 4);
}

hipError_t launch_grouped_gemm(const uint8_t* a_q, const float* a_s, const int32_t* a_rows,
                               const int32_t* group_offset, int G, int64_t M_total,
                               const uint8_t* b_q, const float* b_s, int N, int K, int epi,
                               float* out, uint8_t* out_q, float* out_s, void* ws,
                               hipStream_t st) {
    int32_t* ts = static_cast<int32_t*>(ws);
    int4* tiles = reinterpret_cast<int4*>(static_cast<char*>(ws) + tile_list_offset(G));
    float* a_sT = reinterpret_cast<float*>(static_cast<char*>(ws) + scale_copy_offset(G, M_total, N));
    const int ns = K / BK;
    // 32-row tiles when the groups average at most 64 rows (few tokens per expert)
    const int bm = (M_total <= (int64_t)64 * G) ? 32 : 128;
    const int64_t list_bound = ((M_total + bm - 1) / bm + G) * (int64_t)((N + BN - 1) / BN);
    const int64_t nl = (list_bound + 255) / 256, ng = (M_total + 63) / 64;
    if (G <= PREP_MAX_G) {
        hipLaunchKernelGGL(gemm_prep_kernel, dim3((unsigned)(nl + ng)), dim3(256), 0, st, group_offset, G, bm, N,
                           (int)nl, ts, tiles, a_s, a_rows, M_total, ns, a_sT);
    } else {
        hipLaunchKernelGGL(gemm_scale_gather_kernel, dim3((unsigned)ng), dim3(256), 0, st,
                           a_s, a_rows, M_total, ns, a_sT);
        hipLaunchKernelGGL(gemm_tile_map_kernel, dim3(1), dim3(256), 0, st, group_offset, G, bm, ts);
        hipLaunchKernelGGL(gemm_tile_list_kernel, dim3((unsigned)nl), dim3(256), 0, st,
                           group_offset, ts, G, bm, N, tiles);
    }
    GemmArgs p{a_q, a_sT, (uint32_t)(M_total * 4), a_rows, group_offset, ts, ts + G + 1, tiles, G, b_q, b_s, N, K,
               out, out_q, out_s};
    const int64_t blocks = list_bound;
    // one block per CU (its ~150 KB of LDS admit one), a multiple of the 8 XCDs
    const int64_t persistent = ((int64_t)cu_count_for_current_device() + 7) / 8 * 8;
    const int64_t needed = (blocks + 7) / 8 * 8;
    dim3 grid((unsigned)(needed < persistent ? needed : persistent));
#define MOE_LAUNCH(K, E, B) hipLaunchKernelGGL((K<E, B>), grid, dim3(NT), 0, st, p)
    // The ring kernel (no pipeline restart between tiles) for 128-row tiles of
    // at most 16 slices, where that restart is a large share of a tile: it
    // measured 5% faster on the expert down-projection (K = 2048) and 1-5%
    // slower on tiles of 32 or more slices and on 32-row tiles.  It needs four
    // slices to fetch the next tile's rows ahead, and one tile's rows of the
    // output below 2 GiB (its out-of-range store offsets have bit 31 set).
    const bool ring = bm == 128 && ns >= RING_MIN_SLICES && ns <= 16 &&
                      (int64_t)128 * N * 4 < ((int64_t)1 << 31);
    if (bm == 32) {
        switch (epi) {
            case EPI_STORE_F32: MOE_LAUNCH(grouped_gemm_kernel, EPI_STORE_F32, 32); break;
            case EPI_SWIGLU_F32: MOE_LAUNCH(grouped_gemm_kernel, EPI_SWIGLU_F32, 32); break;
            case EPI_SWIGLU_QUANT_Z: MOE_LAUNCH(grouped_gemm_kernel, EPI_SWIGLU_QUANT_Z, 32); break;
            default: MOE_LAUNCH(grouped_gemm_kernel, EPI_SWIGLU_QUANT, 32); break;
        }
    } else if (ring) {
        switch (epi) {
            case EPI_STORE_F32: MOE_LAUNCH(grouped_gemm_ring_kernel, EPI_STORE_F32, 128); break;
            case EPI_SWIGLU_F32: MOE_LAUNCH(grouped_gemm_ring_kernel, EPI_SWIGLU_F32, 128); break;
            case EPI_SWIGLU_QUANT_Z: MOE_LAUNCH(grouped_gemm_ring_kernel, EPI_SWIGLU_QUANT_Z, 128); break;
            default: MOE_LAUNCH(grouped_gemm_ring_kernel, EPI_SWIGLU_QUANT, 128); break;
        }
    } else {
        switch (epi) {
            case EPI_STORE_F32: MOE_LAUNCH(grouped_gemm_kernel, EPI_STORE_F32, 128); break;
            case EPI_SWIGLU_F32: MOE_LAUNCH(grouped_gemm_kernel, EPI_SWIGLU_F32, 128); break;
            case EPI_SWIGLU_QUANT_Z: MOE_LAUNCH(grouped_gemm_kernel, EPI_SWIGLU_QUANT_Z, 128); break;
            default: MOE_LAUNCH(grouped_gemm_kernel, EPI_SWIGLU_QUANT, 128); break;
        }
    }
#undef MOE_LAUNCH
    return hipGetLastError();
}

// ---- static scratch of the allocation-free GEMM entry point.  Each GPU the
// library runs on holds its own copy of this array (the tile map, tile list
// and slice-major A scales of one call) from module load until the process
// ends.  In host code `scratch` only names the symbol: kernels get the
// device address hipGetSymbolAddress returns, looked up once per device.
static __device__ __attribute__((aligned(256))) unsigned char scratch[MOE_GEMM_SCRATCH_BYTES];

hipError_t gemm_static_scratch(void** ptr) {
    static std::atomic<void*> addr[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {          // first call on this device (a lost race repeats the lookup)
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return hipSuccess;
}

namespace {
// go[g] = g * rows for g = 0..G: the row offsets of G groups of equal height
__global__ __launch_bounds__(256) void equal_groups_kernel(int32_t* __restrict__ go, int G, int rows) {
    for (int g = blockIdx.x * 256 + threadIdx.x; g <= G; g += gridDim.x * 256) go[g] = g * rows;
}
int64_t equal_groups_bytes(int G) { return ((int64_t)(G + 1) * 4 + 255) / 256 * 256; }
}  // namespace

size_t gemm_kgrouped_ws_bytes(int G, int rows, int N) {
    return (size_t)(equal_groups_bytes(G) + scale_copy_offset(G, (int64_t)G * rows, N));
}

hipError_t launch_grouped_gemm_kgrouped(const uint8_t* a_q, const float* a_s, const int32_t* kb_start, int G,
                                        int rows, const uint8_t* b_q, const float* b_s, int b_cs, int N,
                                        float* out, void* ws, hipStream_t st) {
    int32_t* go = static_cast<int32_t*>(ws);
    char* gws = static_cast<char*>(ws) + equal_groups_bytes(G);
    int32_t* ts = reinterpret_cast<int32_t*>(gws);
    int4* tiles = reinterpret_cast<int4*>(gws + tile_list_offset(G));
    const int64_t M_total = (int64_t)G * rows;
    const int bm = 128;
    hipLaunchKernelGGL(equal_groups_kernel, dim3((unsigned)((G + 256) / 256)), dim3(256), 0, st, go, G, rows);
    const int64_t list_bound = ((M_total + bm - 1) / bm + G) * (int64_t)((N + BN - 1) / BN);
    const int64_t nl = (list_bound + 255) / 256;
    if (G <= PREP_MAX_G) {
        // the tile-list blocks only: the A scales are read in place
        hipLaunchKernelGGL(gemm_prep_kernel, dim3((unsigned)nl), dim3(256), 0, st, go, G, bm, N, (int)nl, ts, tiles,
                           nullptr, nullptr, M_total, 1, nullptr);
    } else {
        hipLaunchKernelGGL(gemm_tile_map_kernel, dim3(1), dim3(256), 0, st, go, G, bm, ts);
        hipLaunchKernelGGL(gemm_tile_list_kernel, dim3((unsigned)nl), dim3(256), 0, st, go, ts, G, bm, N, tiles);
    }
    GemmArgs p{a_q, a_s, 0u, nullptr, go, ts, ts + G + 1, tiles, G, b_q, b_s, N, BK,
               out, nullptr, nullptr, kb_start, rows, b_cs};
    const int64_t persistent = ((int64_t)cu_count_for_current_device() + 7) / 8 * 8;
    const int64_t needed = (list_bound + 7) / 8 * 8;
    hipLaunchKernelGGL((grouped_gemm_kernel<EPI_STORE_F32, 128, true>),
                       dim3((unsigned)(needed < persistent ? needed : persistent)), dim3(NT), 0, st, p);
    return hipGetLastError();
}

}  // namespace moe
