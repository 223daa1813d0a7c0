// Direct-to-LDS MFMA mainloop (gfx950) shared by both GEMM kernels of the chain.
//
// Block tile BM x BN, NW waves in a WAVES_M x WAVES_N grid, each wave owning a sub-tile
// made of 32x32 MFMA blocks.  A k-tile is RB bytes of every row (RB = 64: 32 bf16 / 64
// e4m3 values; RB = 128: 64 bf16 / 128 e4m3).
//
// Global -> LDS: `buffer_load_dwordx4 ... lds` moves 16 bytes per lane straight into
// LDS (no VGPR staging).  One instruction fills 1 KB = 1024/RB consecutive panel rows:
// lane i lands at LDS byte 16*i of that 1 KB, i.e. row i / (RB/16), slot i % (RB/16).
//
// LDS layout: 16-byte chunk c of row r sits in a swizzled slot (swz below).  The LDS has
// 64 banks (256 bytes) and serves a ds_read_b128 16 lanes at a time; the 16 lanes of a
// fragment read touch 16 consecutive rows at one chunk, and the swizzle spreads them over
// all 16 distinct 16-byte bank groups:  RB = 64: slot = c ^ ((r >> 2) & 3);  RB = 128:
// slot = c ^ ((r >> 1) & 7).  On the DMA side each lane therefore FETCHES the chunk that
// belongs in the slot it lands in.
//
// Rows past the matrix and chunks past K read as zero through the buffer descriptor's
// range check (each descriptor spans exactly the valid rows of one row segment; K-tail
// chunks get an offset beyond every range).
//
// Pipeline: NS LDS stages; the DMA of tile kt+NS is issued once tile kt has been read
// (details at mainloop_dma).
#pragma once

#include <type_traits>
#include <utility>

#include "device_common.hpp"

namespace coda {

// Operand element kinds and their sizes.
enum class Elt { BF16, E4M3 };
template <Elt E> struct EltInfo;
template <> struct EltInfo<Elt::BF16> { static constexpr int kBytes = 2; };
template <> struct EltInfo<Elt::E4M3> { static constexpr int kBytes = 1; };

constexpr uint32_t kOob = 0x80000000u;  // offset that no descriptor range reaches

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS byte offset of 16-byte chunk `chunk` of panel row `row` (RB bytes per row).
template <int RB>
__device__ __forceinline__ int swz(int row, int chunk) {
    static_assert(RB == 64 || RB == 128, "row depth");
    if constexpr (RB == 64) return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
    return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor of [base, base + bytes) as four SGPRs: base address (48 bits, stride
// 0), num_records = bytes (range-checked), dword3 0x00020000 (raw untyped buffer, 32-bit
// data format).  The fields are made explicitly wave-uniform (readfirstlane).
__device__ __forceinline__ u32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    u32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32)) & 0xFFFFu;
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// One global -> LDS DMA instruction: 16 bytes per lane from rsrc + voff into LDS at
// lds_base + 16 * lane.  Written as inline asm on purpose: the compiler then does not
// track it, so it cannot insert the conservative "wait for every LDS DMA" it would place
// before the next LDS read (it cannot tell that the DMA targets another stage).  The
// caller orders it explicitly with s_waitcnt vmcnt and barriers.
__device__ __forceinline__ void dma16(const u32x4_t& rsrc, uint32_t voff, uint32_t lds_base) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base));
}

__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// One operand panel of R rows, made of up to two row segments (the SwiGLU weight panel
// takes its first SPLIT rows from the gate rows and the rest from the up rows; SPLIT == R
// for a single segment), loaded by NW waves.  Instruction j of wave w covers panel rows
// [(NW*j + w) * RPI, +RPI) with RPI = 1024/RB rows per instruction, so with
// SPLIT % (RPI*NW) == 0 every instruction stays inside one segment and the segment of
// instruction j is j < SPLIT/(RPI*NW).
template <int R, int SPLIT, int NW, int RB>
struct DmaPanel {
    static constexpr int kCpr = RB / 16;            // 16-byte chunks per row
    static constexpr int kRpi = 1024 / RB;          // rows per instruction (one wave)
    static constexpr int kRowsPerInst = kRpi * NW;  // rows per instruction index, all waves
    static_assert(R % kRowsPerInst == 0 && SPLIT % kRowsPerInst == 0 && SPLIT <= R, "panel geometry");
    static_assert(RB == 64 || NW % 2 == 0, "RB = 128 swizzle phase needs an even wave count");
    static constexpr int kInst = R / kRowsPerInst;  // DMA instructions per wave per k-tile
    static constexpr int kSplitInst = SPLIT / kRowsPerInst;
    u32x4_t rsrc[2];
    uint32_t off0;            // byte offset of this lane's chunk in instruction 0 at k-tile 0
    uint32_t chunk_byte;      // 16 * the chunk this lane fetches
    uint32_t stride;          // bytes between instruction j and j+1, wave-uniform

    // seg_base[s]: address of the segment's first row; seg_rows[s]: rows of the segment that
    // exist in the matrix (the descriptor range); kbytes: bytes of one matrix row.
    __device__ __forceinline__ void init(const uint8_t* seg_base0, int seg_rows0,
                                         const uint8_t* seg_base1, int seg_rows1, int kbytes) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rsrc[0] = make_rsrc(seg_base0, static_cast<uint32_t>(max(seg_rows0, 0)) * kbytes);
        rsrc[1] = make_rsrc(seg_base1, static_cast<uint32_t>(max(seg_rows1, 0)) * kbytes);
        // lane lands in row r = row0 + lane/kCpr, slot lane%kCpr; it fetches the chunk that
        // swz<RB> places in that slot.  The swizzle phase of r does not depend on the
        // instruction index j (row0 = (NW*j + wave) * kRpi).
        const int r = wave * kRpi + lane / kCpr;
        const int slot = lane % kCpr;
        const int chunk = (RB == 64) ? (slot ^ ((r >> 2) & 3)) : (slot ^ ((r >> 1) & 7));
        chunk_byte = static_cast<uint32_t>(chunk) << 4;
        off0 = static_cast<uint32_t>(r) * kbytes + chunk_byte;
        stride = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kRowsPerInst) * static_cast<uint32_t>(kbytes));
    }

    // Offset of this lane's chunk for k-tile kt (kOob past K): a chunk past K starts from
    // kOob, and kOob + jj*stride stays beyond every range (each descriptor spans < 2^31
    // bytes), so the whole lane reads zeros.
    __device__ __forceinline__ uint32_t base_offset(int kt, int kbytes) const {
        const uint32_t kb = static_cast<uint32_t>(kt) * RB;
        const bool kin = kb + chunk_byte < static_cast<uint32_t>(kbytes);
        uint32_t base = kin ? off0 + kb : kOob;
        // keep the per-instruction offsets derived at their use (not kInst live registers)
        asm volatile("" : "+v"(base));
        return base;
    }
    // DMA instruction j of k-tile (base from base_offset) into `stage` (R rows x RB bytes).
    // Row of instruction j, lane l: (NW*j + wave) * kRpi + l/kCpr; segment-1 rows are
    // rebased by SPLIT.
    __device__ __forceinline__ void issue_one(int j, uint8_t* stage, uint32_t base) const {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int row0 = (NW * j + wave) * kRpi;
        const int jj = (j < kSplitInst) ? j : j - kSplitInst;
        dma16(rsrc[(j < kSplitInst) ? 0 : 1], base + static_cast<uint32_t>(jj) * stride,
              lds_addr(stage + row0 * RB));
    }
    // All kInst instructions of k-tile kt.
    __device__ __forceinline__ void issue(uint8_t* stage, int kt, int kbytes) const {
        const uint32_t base = base_offset(kt, kbytes);
#pragma unroll
        for (int j = 0; j < kInst; ++j) issue_one(j, stage, base);
    }
};

// Fragments of one MFMA k-step for a wave's TM x TN 32x32 blocks.  bf16: a k-step is
// k16 (RB/32 per k-tile), one 16-byte ds_read per fragment.  e4m3: a k-step is k64
// (RB/64 per k-tile), two 16-byte ds_reads per fragment.
// TC: the MFMA takes the B fragment as its first operand, so each 32x32 accumulator
// block holds the transposed product (lane = A row, registers = B rows); the operand
// layouts are the same, only the roles swap.
template <Elt E, int TM, int TN, int RB, bool TC = false>
struct Frags;

template <int TM, int TN, int RB, bool TC>
struct Frags<Elt::BF16, TM, TN, RB, TC> {
    static constexpr int kSteps = RB / 32;
    static constexpr int kReads = TM + TN;         // ds_read_b128 per k-step
    bf16x8_t a[TM], b[TN];
    // fragment read i of k-step s, in the order the k-step's MFMAs first use them
    // (MFMA j uses a[j / TN] and b[j % TN]): a[0], b[0..TN-1], a[1..TM-1]
    template <class ARow, class BRow>
    __device__ __forceinline__ void load_one(int i, const uint8_t* sA, const uint8_t* sB, int s,
                                             const ARow& a_row, const BRow& b_row) {
        const int lane = threadIdx.x & 63;
        const int lr = lane & 31, lh = lane >> 5;
        if (i == 0)
            a[0] = *reinterpret_cast<const bf16x8_t*>(sA + swz<RB>(a_row(0) + lr, 2 * s + lh));
        else if (i <= TN)
            b[i - 1] = *reinterpret_cast<const bf16x8_t*>(sB + swz<RB>(b_row(i - 1) + lr, 2 * s + lh));
        else
            a[i - TN] = *reinterpret_cast<const bf16x8_t*>(sA + swz<RB>(a_row(i - TN) + lr, 2 * s + lh));
    }
    template <class ARow, class BRow>
    __device__ __forceinline__ void load(const uint8_t* sA, const uint8_t* sB, int s,
                                         const ARow& a_row, const BRow& b_row) {
#pragma unroll
        for (int i = 0; i < kReads; ++i) load_one(i, sA, sB, s, a_row, b_row);
    }
    // MFMA i of the k-step: block (i / TN, i % TN); Z: the block starts from zero (the
    // MFMA's C operand is the inline constant 0, so the block needs no zeroing before)
    template <bool Z = false>
    __device__ __forceinline__ void mma_one(int i, f32x16_t (&acc)[TM][TN]) const {
        const int tm = i / TN, tn = i % TN;
        const f32x16_t c = Z ? f32x16_t{} : acc[tm][tn];
        if constexpr (TC)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[tn], a[tm], c, 0, 0, 0);
        else
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tm], b[tn], c, 0, 0, 0);
    }
    __device__ __forceinline__ void mma(f32x16_t (&acc)[TM][TN]) const {
#pragma unroll
        for (int i = 0; i < TM * TN; ++i) mma_one(i, acc);
    }
};

template <int TM, int TN, int RB>
struct Frags<Elt::E4M3, TM, TN, RB, false> {
    static constexpr int kSteps = RB / 64;
    static constexpr int kReads = TM + TN;         // fragments (two ds_read_b128 each)
    i32x8_t a[TM], b[TN];
    // fragment i of k-step s (lane holds 32 bytes of its row = chunks 4s + 2*lh, +1), in
    // the order the k-step's MFMAs first use them: a[0], b[0..TN-1], a[1..TM-1]
    template <class ARow, class BRow>
    __device__ __forceinline__ void load_one(int i, const uint8_t* sA, const uint8_t* sB, int s,
                                             const ARow& a_row, const BRow& b_row) {
        const int lane = threadIdx.x & 63;
        const int lr = lane & 31, lh = lane >> 5;
        const bool isa = i == 0 || i > TN;
        const int idx = i == 0 ? 0 : (i <= TN ? i - 1 : i - TN);
        const int row = (isa ? a_row(idx) : b_row(idx)) + lr;
        const uint8_t* base = isa ? sA : sB;
        const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + swz<RB>(row, 4 * s + 2 * lh));
        const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + swz<RB>(row, 4 * s + 2 * lh + 1));
        const i32x8_t v = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (isa) a[idx] = v; else b[idx] = v;
    }
    template <class ARow, class BRow>
    __device__ __forceinline__ void load(const uint8_t* sA, const uint8_t* sB, int s,
                                         const ARow& a_row, const BRow& b_row) {
#pragma unroll
        for (int i = 0; i < kReads; ++i) load_one(i, sA, sB, s, a_row, b_row);
    }
    template <bool Z = false>
    __device__ __forceinline__ void mma_one(int i, f32x16_t (&acc)[TM][TN]) const {
        const int tm = i / TN, tn = i % TN;
        // formats 0/0 = e4m3 x e4m3; block scales 127 = 2^0 (unscaled)
        acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[tm], b[tn], Z ? f32x16_t{} : acc[tm][tn],
                                                                      0, 0, 0, 127, 0, 127);
    }
    __device__ __forceinline__ void mma(f32x16_t (&acc)[TM][TN]) const {
#pragma unroll
        for (int i = 0; i < TM * TN; ++i) mma_one(i, acc);
    }
};

// ---------------------------------------------------------------------------------
// Token-major operands (the weight gradients, whose contraction runs over the tokens of
// row-major activations: G[j,k] = sum_m X[m,j] Y[m,k]).  A panel is 256 columns (512
// bytes) of 64 consecutive token rows per k-tile; in LDS each token row is 512 bytes with
// its 16-byte chunks XOR-swizzled by (token row mod 4) * 4, applied on the global side so
// the DMA writes stay linear.  Fragments come from LDS transpose reads
// (ds_read_b64_tr_b16): within each 16-lane group, lane L reads 4 consecutive columns of
// token row L / 4, and lane i receives column i of those 4 token rows, i.e. 4 consecutive
// k of one MFMA row; two reads give the 8 k a 32x32x16 fragment lane holds.  With the
// swizzle the 4 token rows of a read land in 4 different 16-bank groups.
// A k-tile's address of one lane's chunk in a token-major panel: a descriptor of that
// k-tile's 64 token rows alone (rebased on every k-tile, so operands larger than 4 GB
// need no 64-bit offsets) and the lane's offset inside it.
struct TokAddr {
    u32x4_t rsrc;
    uint32_t voff;
};

template <int NW>
struct DmaPanelTok {
    static constexpr int kTok = 64;                   // tokens per k-tile
    static constexpr int kRowBytes = 512;             // 256 bf16 columns
    static constexpr int kRowsPerInst = 2 * NW;       // token rows per instruction index
    static constexpr int kInst = kTok / kRowsPerInst; // DMA instructions per wave per k-tile
    static_assert(NW % 2 == 0, "a lane's token row phase (mod 4) must not depend on the instruction");
    const uint8_t* base;  // the panel's first column in token row 0 of the range
    int tokens;           // token rows in the range
    uint32_t ld;          // bytes between token rows
    uint32_t off0;        // byte offset of this lane's chunk in instruction 0 of a k-tile
    uint32_t stride;      // bytes between instruction j and j + 1
    bool col_in;          // this lane's chunk lies inside the matrix's columns

    // base: the panel's first column in token row 0 (of the range); tokens: token rows in
    // range from base (rows past them read zeros); ld: bytes between token rows (64 rows
    // of it must stay below 2^31); cols: columns of the panel inside the matrix (chunks
    // past them read zeros).
    __device__ __forceinline__ void init(const uint8_t* base_, int tokens_, int ld_, int cols) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int r = 2 * wave + (lane >> 5);          // token row in instruction 0
        const int p = lane & 31;                       // chunk position in the LDS row
        const int c = p ^ ((r & 3) << 2);              // chunk of the matrix row it holds
        col_in = c * 8 < cols;
        base = base_;
        tokens = __builtin_amdgcn_readfirstlane(max(tokens_, 0));
        ld = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(ld_));
        off0 = static_cast<uint32_t>(r) * ld + static_cast<uint32_t>(c) * 16;
        stride = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kRowsPerInst) * ld);
    }
    // k-tile kt: a descriptor of its token rows inside the range (none past the range:
    // reads of zeros) and this lane's chunk offset (kOob for a chunk past the columns)
    __device__ __forceinline__ TokAddr base_offset(int kt, int /*kbytes*/) const {
        const int rows = min(max(tokens - kt * kTok, 0), kTok);
        TokAddr a;
        a.rsrc = make_rsrc(base + static_cast<uint64_t>(kt) * kTok * ld, static_cast<uint32_t>(rows) * ld);
        uint32_t v = col_in ? off0 : kOob;
        asm volatile("" : "+v"(v));
        a.voff = v;
        return a;
    }
    __device__ __forceinline__ void issue_one(int j, uint8_t* stage, const TokAddr& a) const {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        dma16(a.rsrc, a.voff + static_cast<uint32_t>(j) * stride, lds_addr(stage + (2 * (NW * j + wave)) * kRowBytes));
    }
    __device__ __forceinline__ void issue(uint8_t* stage, int kt, int kbytes) const {
        const TokAddr a = base_offset(kt, kbytes);
#pragma unroll
        for (int j = 0; j < kInst; ++j) issue_one(j, stage, a);
    }
};

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// Fragments of 32x32x16 bf16 MFMAs from token-major LDS panels (DmaPanelTok layout):
// k-step s covers tokens 16 s .. 16 s + 15 of the k-tile; a_row / b_row give the first
// panel column of a block (a multiple of 32).
template <int TM, int TN>
struct FragsTok {
    static constexpr int kSteps = DmaPanelTok<2>::kTok / 16;
    static constexpr int kReads = TM + TN;
    bf16x8_t a[TM], b[TN];
    __device__ __forceinline__ static bf16x8_t read(const uint8_t* panel, int col0, int s) {
        const int lane = threadIdx.x & 63;
        const int g = lane >> 4, L = lane & 15;
        const int col = col0 + 16 * (g & 1) + 4 * (L & 3);
        i16x4_t v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tt = 16 * s + 8 * (g >> 1) + 4 * h + (L >> 2);
            const int off = tt * DmaPanelTok<2>::kRowBytes + (((col >> 3) ^ ((tt & 3) << 2)) << 4) + (col & 7) * 2;
            v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4_t*)((__attribute__((address_space(3))) uint8_t*)(lds_ptr_t)panel + off));
        }
        const i16x4_t lo = v[0], hi = v[1];
        return __builtin_bit_cast(bf16x8_t, (short __attribute__((ext_vector_type(8)))){
            lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
    template <class ARow, class BRow>
    __device__ __forceinline__ void load_one(int i, const uint8_t* sA, const uint8_t* sB, int s,
                                             const ARow& a_row, const BRow& b_row) {
        if (i == 0)
            a[0] = read(sA, a_row(0), s);
        else if (i <= TN)
            b[i - 1] = read(sB, b_row(i - 1), s);
        else
            a[i - TN] = read(sA, a_row(i - TN), s);
    }
    template <class ARow, class BRow>
    __device__ __forceinline__ void load(const uint8_t* sA, const uint8_t* sB, int s,
                                         const ARow& a_row, const BRow& b_row) {
#pragma unroll
        for (int i = 0; i < kReads; ++i) load_one(i, sA, sB, s, a_row, b_row);
    }
    template <bool Z = false>
    __device__ __forceinline__ void mma_one(int i, f32x16_t (&acc)[TM][TN]) const {
        const int tm = i / TN, tn = i % TN;
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tm], b[tn], Z ? f32x16_t{} : acc[tm][tn], 0, 0, 0);
    }
};

// Compile-time loop: f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// The fragments of two consecutive k-steps (parity p = k-step & 1), as the mainloop
// drives them: mma_one(p, j) is MFMA j of a k-step, slot<J>(p, ...) the LDS work of slot
// J that prepares the next k-step (here: fragment read J).
template <class F>
struct FragPair {
    static constexpr int kSteps = F::kSteps;
    F f[2];
    template <int J, class ARow, class BRow>
    __device__ __forceinline__ void slot(int p, const uint8_t* sA, const uint8_t* sB, int s,
                                         const ARow& a_row, const BRow& b_row) {
        if constexpr (J < F::kReads) f[p].load_one(J, sA, sB, s, a_row, b_row);
    }
    template <class ARow, class BRow>
    __device__ __forceinline__ void load(int p, const uint8_t* sA, const uint8_t* sB, int s,
                                         const ARow& a_row, const BRow& b_row) {
        f[p].load(sA, sB, s, a_row, b_row);
    }
    template <bool Z = false, int TM, int TN>
    __device__ __forceinline__ void mma_one(int p, int j, f32x16_t (&acc)[TM][TN]) const {
        f[p].template mma_one<Z>(j, acc);
    }
};

// bf16 activations x e4m3 weights (weight-only 8-bit), bf16 MFMA.  A panel: 128-byte
// rows (64 bf16 per k-tile); B panel: 64-byte rows (64 e4m3 per k-tile), kept as e4m3 in
// LDS and converted exactly to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8, scale 1).
//
// k order inside a 64-k tile: k-step s = 2t + h gives lane half lh the k values
// 32t + 16lh + 8h + (0..7) of BOTH operands, i.e. A chunk 4t + 2lh + h of its row and
// bytes 8h .. 8h+7 of B chunk 2t + lh.  Each k-step still sums over 16 distinct k, so the
// tile computes the plain product; one 16-byte B read per lane serves two k-steps.
//
// Slots of the k-step before step s (parity p = s & 1): A reads in slots 0 .. TM-1; for
// an even s the raw B reads in slots TM .. TM+TN-1 and the conversion of their low halves
// in the last TN slots (the reads have had the slots in between to land); for an odd s
// the conversion of the high halves of the same raw chunks.
template <int TM, int TN>
struct FragsW8 {
    static constexpr int kSteps = 4;
    static constexpr int kRbA = 128, kRbB = 64;
    static constexpr int kMfma = TM * TN;
    static_assert(TM + 2 * TN <= kMfma, "reads and conversions fit the MFMA slots");
    bf16x8_t a[2][TM], b[2][TN];
    i32x4_t raw[TN];

    __device__ __forceinline__ static bf16x8_t cvt8(int w0, int w1) {
        typedef int i32x4v __attribute__((ext_vector_type(4)));
        const i32x4v q = {__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                          __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                          __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                          __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
        return __builtin_bit_cast(bf16x8_t, q);
    }
    template <int J, class ARow, class BRow>
    __device__ __forceinline__ void slot(int p, const uint8_t* sA, const uint8_t* sB, int s,
                                         const ARow& a_row, const BRow& b_row) {
        const int lane = threadIdx.x & 63;
        const int lr = lane & 31, lh = lane >> 5;
        const int t = s >> 1, h = s & 1;
        if constexpr (J < TM) {
            a[p][J] = *reinterpret_cast<const bf16x8_t*>(sA + swz<kRbA>(a_row(J) + lr, 4 * t + 2 * lh + h));
        } else if constexpr (J < TM + TN) {
            if (h == 0)
                raw[J - TM] = *reinterpret_cast<const i32x4_t*>(sB + swz<kRbB>(b_row(J - TM) + lr, 2 * t + lh));
        }
        if constexpr (J >= kMfma - TN) {
            constexpr int tn = J - (kMfma - TN);
            b[p][tn] = h == 0 ? cvt8(raw[tn][0], raw[tn][1]) : cvt8(raw[tn][2], raw[tn][3]);
        }
    }
    template <class ARow, class BRow>
    __device__ __forceinline__ void load(int p, const uint8_t* sA, const uint8_t* sB, int s,
                                         const ARow& a_row, const BRow& b_row) {
        static_for<kMfma>([&](auto J) { slot<decltype(J)::value>(p, sA, sB, s, a_row, b_row); });
    }
    template <bool Z = false>
    __device__ __forceinline__ void mma_one(int p, int i, f32x16_t (&acc)[TM][TN]) const {
        const int tm = i / TN, tn = i % TN;
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[p][tm], b[p][tn], Z ? f32x16_t{} : acc[tm][tn],
                                                              0, 0, 0);
    }
};

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14]); expcnt / lgkmcnt are left at their maxima.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }


// The whole mainloop: acc += A_panel . B_panel^T over the k-tiles of one row.
// st[0..NS-1] are the NS stage buffers, each (BM + BN) * RB bytes.
//
// Software pipeline (per wave).  Fragments are double-buffered by MFMA k-step: the
// fragments of step j+1 are read from LDS while the MFMAs of step j run.  The last
// k-step of tile kt is where tile kt+1's first fragments are needed; its MFMAs only use
// fragments already in registers, so every LDS read of tile kt has been issued before it.
// There the wave waits for tile kt+1's DMA and passes the barrier; after it every wave
// has finished reading tile kt, so tile kt's stage receives the DMA of tile kt+NS, issued
// (one instruction per MFMA) together with the reads of tile kt+1's first fragments.
// The DMA thus runs NS tiles ahead of the reads, and tiles kt+2 .. kt+NS-1 may still be
// in flight at the barrier of tile kt.
//
// SPREAD (1 .. k-steps per tile) spreads the DMA of tile kt+NS over SPREAD k-steps: the
// last k-step of tile kt and the first SPREAD-1 k-steps of tile kt+1, at most
// ceil(kPerTile / SPREAD) instructions per k-step.  A wave whose DMA instructions back up
// in the memory pipeline stops issuing MFMAs too, so a burst of them in one k-step
// stalls the wave and skews it against the others at the next barrier.  Every
// instruction of tile kt+NS is still issued before the last k-step of tile kt+1, so the
// wait counts above hold unchanged.  The prologue issues tile NS-1 the same way (its
// first share up front, the rest during tile 0).
//
// FP provides the fragments (FragPair<Frags<...>> or FragsW8); RBA / RBB are the row
// bytes of one k-tile in the A and B panels (a stage holds BM*RBA + BN*RBB bytes, B
// after A).  kbytes is the byte length of an A row (k-tile count = ceil(kbytes / RBA));
// the B panel's descriptor and K-tail checks use its own row length, set at init.
// The pending DMA of k-tile NS-1 (its base offsets) between the prologue and the run.
// LATER: loads the caller issues after the prologue and before the run (for instance the
// next tile's row scales), which the run's first wait may leave in flight.  Every wave
// must issue exactly LATER such loads (no load skipped behind a branch), else the wait
// would let k-tile 0's DMA still be in flight.
template <class OA, class OB, int LATER = 0>
struct DmaPending {
    static constexpr int kLater = LATER;
    OA a;
    OB b;
};

// Compile-time schedule constants of mainloop_dma_fp.
template <class FP, int NS, int SPREAD, int TM, int TN, class PA, class PB>
struct DmaSched {
    static constexpr int KS = FP::kSteps;
    static constexpr int kMfma = TM * TN;
    static constexpr int nA = PA::kInst;
    static constexpr int kPerTile = nA + PB::kInst;                        // DMA per wave per tile
    static constexpr int kPer = (kPerTile + SPREAD - 1) / SPREAD;          // DMA per k-step
    // the continuous mainloop (mainloop_dma_cont): kPer0 instructions at the crossing, the
    // rest kPerS per k-step over the next SPREAD-1 k-steps
#ifdef CODA_CONT_D0
    static constexpr int kPer0 = CODA_CONT_D0 < kPerTile ? CODA_CONT_D0 : kPerTile;
#else
    static constexpr int kPer0 = kPer;
#endif
    static constexpr int kPerS = SPREAD > 1 ? (kPerTile - kPer0 + SPREAD - 2) / (SPREAD - 1) : 0;
    static_assert(NS >= 2, "at least two stages");
    static_assert((NS * KS) % 2 == 0, "fragment double-buffer parity must repeat every stage group");
    static_assert((NS - 1) * kPerTile < 64, "vmcnt range");
    static_assert(SPREAD >= 1 && SPREAD <= KS, "the DMA of a tile ends before the next tile's last k-step");
    static_assert(kPer <= kMfma && kPer0 <= kMfma && kPerS <= kMfma, "one MFMA ahead of every DMA instruction");
    static_assert(SPREAD > 1 || kPer0 == kPerTile, "without a spread the crossing issues the whole k-tile");
};

// Prologue of the pipelined mainloop: the DMA of k-tiles 0 .. NS-2 and the first share of
// k-tile NS-1, nothing waited for.  Issued on its own (mainloop_dma_run follows), it lets
// a caller that owns the LDS stages start the next tile's loads before other work (a
// persistent kernel's epilogue that does not touch the LDS).
template <class FP, int BM, int NS, int RBA, int SPREAD, int TM, int TN, class PA, class PB>
__device__ __forceinline__ auto mainloop_dma_prologue(const PA& pa, const PB& pb, int kbytes, int kbytes_b,
                                                      uint8_t* const (&st)[NS]) {
    using D = DmaSched<FP, NS, SPREAD, TM, TN, PA, PB>;
    constexpr int nA = D::nA, kPer = D::kPer;
    constexpr int kOffB = BM * RBA;
    auto issue_q = [&](int q, uint8_t* stage, const auto& ba, const auto& bb) {
        if (q < nA) pa.issue_one(q, stage, ba);
        else pb.issue_one(q - nA, stage + kOffB, bb);
    };
    static_for<NS - 1>([&](auto I) {
        constexpr int i = decltype(I)::value;
        pa.issue(st[i], i, kbytes);
        pb.issue(st[i] + kOffB, i, kbytes_b);
    });
    // tile NS-1: its first share now, the rest as pending DMA during tile 0
    DmaPending<decltype(pa.base_offset(0, kbytes)), decltype(pb.base_offset(0, kbytes_b))> pend{
        pa.base_offset(NS - 1, kbytes), pb.base_offset(NS - 1, kbytes_b)};
    static_for<kPer>([&](auto Q) { issue_q(decltype(Q)::value, st[NS - 1], pend.a, pend.b); });
    return pend;
}

// mainloop_dma_prologue one instruction at a time, so that a caller can spread it over
// other work (a persistent kernel's epilogue): instruction Q of kOps, in the order the
// prologue issues them (tiles 0 .. NS-2 whole, A panel before B, then the first share of
// tile NS-1).  pending<LATER>() is then what mainloop_dma_prologue would have returned.
template <class FP, int BM, int NS, int RBA, int SPREAD, int TM, int TN, class PA, class PB>
struct DmaPrologue {
    using D = DmaSched<FP, NS, SPREAD, TM, TN, PA, PB>;
    static constexpr int kOps = (NS - 1) * D::kPerTile + D::kPer;
    const PA& pa;
    const PB& pb;
    int kbytes, kbytes_b;
    uint8_t* const (&st)[NS];
    template <int Q>
    __device__ __forceinline__ void issue() const {
        static_assert(Q >= 0 && Q < kOps, "prologue instruction");
        constexpr int i = Q / D::kPerTile, r = Q % D::kPerTile;
        if constexpr (r < D::nA) pa.issue_one(r, st[i], pa.base_offset(i, kbytes));
        else pb.issue_one(r - D::nA, st[i] + BM * RBA, pb.base_offset(i, kbytes_b));
    }
    // instructions [kOps * c / parts, kOps * (c + 1) / parts): share c of `parts`
    template <int C, int PARTS>
    __device__ __forceinline__ void issue_share() const {
        static_for<kOps>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            if constexpr (q * PARTS >= kOps * C && q * PARTS < kOps * (C + 1)) issue<q>();
        });
    }
    template <int LATER>
    __device__ __forceinline__ auto pending() const {
        return DmaPending<decltype(pa.base_offset(0, kbytes)), decltype(pb.base_offset(0, kbytes_b)), LATER>{
            pa.base_offset(NS - 1, kbytes), pb.base_offset(NS - 1, kbytes_b)};
    }
};

// Extra loads a kernel issues once per k-tile of the pipelined mainloop, kOps vector
// memory instructions every k-tile (for instance a prefetch of the epilogue's operand).
// They go out in the k-step after the previous tile's DMA batch is complete, so the
// tile-end wait allows them to be in flight.  NoExtra: none.
struct NoExtra {
    static constexpr int kOps = 0;
    __device__ __forceinline__ void issue(int /*kt*/, int /*nk*/) const {}
    __device__ __forceinline__ void issue_into(int /*kt*/, int /*nk*/, uint8_t* /*stage*/) const {}
};

// The rest of the pipelined mainloop after mainloop_dma_prologue: wait for k-tile 0, the
// k-loop, and the drain of the DMA that ran past the end.  The first wait, vmcnt
// <= (NS-2) kPerTile + kPer + Pend::kLater, is exact when only the prologue's DMA and
// kLater further loads were issued after k-tile 0; other vector memory operations issued
// after the prologue (an epilogue's stores) only make it wait longer: loads complete in
// order, so while any load of k-tile 0 is outstanding, so are all later loads of the
// prologue and the kLater loads after it.
template <class FP, int BM, int BN, int SPLIT, int NS, int NW, int RBA, int RBB, int SPREAD, int TM, int TN,
          class ARow, class BRow, class PA, class PB, class Pend, class X = NoExtra>
__device__ __forceinline__ void mainloop_dma_run(f32x16_t (&acc)[TM][TN], const PA& pa, const PB& pb, int kbytes,
                                                 int kbytes_b, uint8_t* const (&st)[NS], const ARow& a_row,
                                                 const BRow& b_row, const Pend& pend0, const X& xtra = X()) {
    using D = DmaSched<FP, NS, SPREAD, TM, TN, PA, PB>;
    constexpr int KS = D::KS, kMfma = D::kMfma, nA = D::nA, kPerTile = D::kPerTile, kPer = D::kPer;
    const int nk = (kbytes + RBA - 1) / RBA;
    // k-tiles run in groups of NS (one per stage); the count is padded to a multiple of NS
    // with k-tiles past K, which the DMA fills with zeros, and is at least one group (K = 0
    // computes a group of zeros, so acc is always written).  The DMA always runs NS tiles
    // ahead, past the padded end too (zeros into stages that are not read again), so the
    // wait counts are exact on every tile.
    const int ng = max((nk + NS - 1) / NS, 1);
    constexpr int kOffB = BM * RBA;          // B panel offset inside a stage
    FP f;
    auto issue_q = [&](int q, uint8_t* stage, const auto& ba, const auto& bb) {
        if (q < nA) pa.issue_one(q, stage, ba);
        else pb.issue_one(q - nA, stage + kOffB, bb);
    };
    auto pend_a = pend0.a;
    auto pend_b = pend0.b;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * kPerTile + kPer + Pend::kLater));   // tile 0 landed
    __syncthreads();
    f.load(0, st[0], st[0] + kOffB, 0, a_row, b_row);

    // group(First, g): the NS k-tiles of group g.  The first group is peeled: its first
    // k-step's MFMAs take a zero C operand, so acc's contents on entry are never read (the
    // callers' zero fill is dead code and no accumulator is written before the first MFMA).
    auto group = [&](auto FirstC, int g) {
        constexpr bool kFirst = decltype(FirstC)::value;
        static_for<NS>([&](auto I) {
            constexpr int i = decltype(I)::value;
            constexpr int par = (i * KS) & 1;     // k-step s of this tile uses f[(par + s) & 1]
            uint8_t* cur = st[i];
            uint8_t* nxt = st[(i + 1) % NS];
            uint8_t* prv = st[(i + NS - 1) % NS];    // stage receiving the pending DMA
            const int kt = g * NS + i;
            static_for<KS - 1>([&](auto Sc) {
                constexpr int s = decltype(Sc)::value;
                // k-step s: MFMA j, then pending DMA instruction (s+1)*kPer + j, then
                // fragment read j of k-step s+1
                static_for<kMfma>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    f.template mma_one<kFirst && i == 0 && s == 0>((par + s) & 1, j, acc);
                    if constexpr (s + 1 < SPREAD && j < kPer && (s + 1) * kPer + j < kPerTile)
                        issue_q((s + 1) * kPer + j, prv, pend_a, pend_b);
                    f.template slot<j>((par + s + 1) & 1, cur, cur + kOffB, s + 1, a_row, b_row);
                    // the extra loads, after the batch's last instruction
                    if constexpr (X::kOps > 0 && j == kMfma - 1 && s == (SPREAD - 1 < KS - 2 ? SPREAD - 1 : KS - 2))
                        xtra.issue(kt, nk);
                    __builtin_amdgcn_sched_barrier(0);
                });
            });
            // last k-step of the tile: cross into tile kt+1 (the extra loads of this tile
            // may still be in flight)
            __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * kPerTile + X::kOps));  // tile kt+1 landed
            __syncthreads();                                             // ... for every wave
            __builtin_amdgcn_sched_barrier(0);
            pend_a = pa.base_offset(kt + NS, kbytes);
            pend_b = pb.base_offset(kt + NS, kbytes_b);
            // MFMA j, then DMA instruction j of tile kt+NS into this tile's stage (the
            // first kPer; the rest follow in tile kt+1), then fragment read j of tile
            // kt+1's first k-step
            static_assert(KS >= 2, "the tile-crossing k-step is not the first");
            static_for<kMfma>([&](auto J) {
                constexpr int j = decltype(J)::value;
                f.mma_one((par + KS - 1) & 1, j, acc);
                if constexpr (j < kPer) issue_q(j, cur, pend_a, pend_b);
                f.template slot<j>((par + KS) & 1, nxt, nxt + kOffB, 0, a_row, b_row);
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };
    group(std::true_type{}, 0);
    for (int g = 1; g < ng; ++g) group(std::false_type{}, g);
    // drain the DMA that ran past the end before the LDS is reused or released
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
}

// Continuous mainloop of a persistent kernel (two stages): the k-tiles 1 .. nkp-1 of the
// current tile (panels pa, pb), whose k-tile 0 the caller has already multiplied into acc
// (it does so during the previous tile's epilogue), and the first loads of the next tile
// (panels na, nb): the DMA stream does not stop at the tile's end, so the crossings of
// k-tiles nkp-2 and nkp-1 load the next tile's k-tiles 0 and 1 into the stages they free.
// nkp is the k-tile count padded to an even number (k-tile kt lives in stage kt & 1); the
// caller guarantees nkp >= 4.
//
// On entry: k-tile 1 has landed for every wave (the caller waited and passed a barrier
// after issuing its last DMA instruction), the stage of k-tile 0 may still be read by
// other waves.  On return: the next tile's k-tile 0 has landed in stage 0 (every wave
// waited and passed the barrier), f[0] holds its first k-step's fragments, and the DMA of
// its k-tile 1 into stage 1 has issued its first kPer0 instructions; the returned offsets
// are that k-tile's, for the caller to issue instructions kPer0 .. kPerTile-1.
//
// The crossing at the end of k-tile kt waits with vmcnt(0) (with two stages nothing later
// than k-tile kt+1's DMA has been issued but stores and the caller's loads), passes the
// barrier, runs kt's last k-step with the first share of k-tile kt+2's DMA (kPer0
// instructions) and the reads of kt+1's first k-step; the rest of kt+2's DMA goes out during
// kt+1's first SPREAD-1 k-steps (kPerS per k-step).
template <class FP, int BM, int RBA, int SPREAD, int TM, int TN, class ARow, class BRow, class PA, class PB>
__device__ __forceinline__ auto mainloop_dma_cont(f32x16_t (&acc)[TM][TN], FP& f, const PA& pa, const PB& pb,
                                                  const PA& na, const PB& nb, int kbytes, uint8_t* const (&st)[2],
                                                  const ARow& a_row, const BRow& b_row) {
    using D = DmaSched<FP, 2, SPREAD, TM, TN, PA, PB>;
    constexpr int KS = D::KS, kMfma = D::kMfma, nA = D::nA, kPerTile = D::kPerTile;
    constexpr int kPer0 = D::kPer0, kPerS = D::kPerS;
    static_assert(KS % 2 == 0, "fragment parity: k-step 0 of every k-tile uses f[0]");
    constexpr int kOffB = BM * RBA;
    const int nkp = (((kbytes + RBA - 1) / RBA) + 1) & ~1;
    using Off = DmaPending<decltype(pa.base_offset(0, kbytes)), decltype(pb.base_offset(0, kbytes))>;
    auto issue = [&](const PA& A, const PB& B, int q, uint8_t* stage, const Off& o) {
        if (q < nA) A.issue_one(q, stage, o.a);
        else B.issue_one(q - nA, stage + kOffB, o.b);
    };
    // k-steps 0 .. KS-2 of a k-tile in stage S, with the rest of the pending DMA (into the
    // other stage, panels A / B)
    auto steps = [&](auto SC, const PA& A, const PB& B, const Off& o) {
        constexpr int S = decltype(SC)::value;
        uint8_t* cur = st[S];
        uint8_t* oth = st[S ^ 1];
        static_for<KS - 1>([&](auto Sc) {
            constexpr int s = decltype(Sc)::value;
            static_for<kMfma>([&](auto J) {
                constexpr int j = decltype(J)::value;
                f.mma_one(s & 1, j, acc);
                if constexpr (s + 1 < SPREAD && j < kPerS && kPer0 + s * kPerS + j < kPerTile)
                    issue(A, B, kPer0 + s * kPerS + j, oth, o);
                f.template slot<j>((s + 1) & 1, cur, cur + kOffB, s + 1, a_row, b_row);
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };
    // the crossing at the end of the k-tile in stage S (MMA: its last k-step; without, the
    // caller has run it): DMA of k-tile dkt of panels A / B into stage S
    auto crossing = [&](auto SC, auto MmaC, const PA& A, const PB& B, int dkt) {
        constexpr int S = decltype(SC)::value;
        constexpr bool kMma = decltype(MmaC)::value;
        if constexpr (kMma) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));     // k-tile kt+1 landed
        __syncthreads();                                                     // ... for every wave
        __builtin_amdgcn_sched_barrier(0);
        const Off o{A.base_offset(dkt, kbytes), B.base_offset(dkt, kbytes)};
        uint8_t* nxt = st[S ^ 1];
        static_for<kMfma>([&](auto J) {
            constexpr int j = decltype(J)::value;
            if constexpr (kMma) f.mma_one((KS - 1) & 1, j, acc);
            if constexpr (j < kPer0) issue(A, B, j, st[S], o);
            f.template slot<j>(0, nxt, nxt + kOffB, 0, a_row, b_row);
            __builtin_amdgcn_sched_barrier(0);
        });
        return o;
    };
    Off o = crossing(std::integral_constant<int, 0>{}, std::false_type{}, pa, pb, 2);
    int kt = 1;
    for (; kt < nkp - 3; kt += 2) {
        steps(std::integral_constant<int, 1>{}, pa, pb, o);
        o = crossing(std::integral_constant<int, 1>{}, std::true_type{}, pa, pb, kt + 2);
        steps(std::integral_constant<int, 0>{}, pa, pb, o);
        o = crossing(std::integral_constant<int, 0>{}, std::true_type{}, pa, pb, kt + 3);
    }
    // k-tiles nkp-3, nkp-2, nkp-1: the last two crossings load the next tile's k-tiles 0, 1
    steps(std::integral_constant<int, 1>{}, pa, pb, o);
    o = crossing(std::integral_constant<int, 1>{}, std::true_type{}, pa, pb, kt + 2);
    steps(std::integral_constant<int, 0>{}, pa, pb, o);
    o = crossing(std::integral_constant<int, 0>{}, std::true_type{}, na, nb, 0);
    steps(std::integral_constant<int, 1>{}, na, nb, o);
    return crossing(std::integral_constant<int, 1>{}, std::true_type{}, na, nb, 1);
}

template <class FP, int BM, int BN, int SPLIT, int NS, int NW, int RBA, int RBB, int SPREAD, int TM, int TN,
          class ARow, class BRow, class PA, class PB, class X = NoExtra>
__device__ __forceinline__ void mainloop_dma_fp(f32x16_t (&acc)[TM][TN], const PA& pa, const PB& pb, int kbytes,
                                                int kbytes_b, uint8_t* const (&st)[NS],
                                                const ARow& a_row, const BRow& b_row, const X& xtra = X()) {
    const auto pend = mainloop_dma_prologue<FP, BM, NS, RBA, SPREAD, TM, TN>(pa, pb, kbytes, kbytes_b, st);
    mainloop_dma_run<FP, BM, BN, SPLIT, NS, NW, RBA, RBB, SPREAD>(acc, pa, pb, kbytes, kbytes_b, st, a_row, b_row,
                                                                  pend, xtra);
}

// Both operands of one element type E with RB-byte k-tile rows.
template <Elt E, int BM, int BN, int SPLIT, int NS, int NW, int RB, int SPREAD, bool TC = false, int TM, int TN,
          class ARow, class BRow, class X = NoExtra>
__device__ __forceinline__ void mainloop_dma(f32x16_t (&acc)[TM][TN], const DmaPanel<BM, BM, NW, RB>& pa,
                                             const DmaPanel<BN, SPLIT, NW, RB>& pb, int kbytes,
                                             uint8_t* const (&st)[NS], const ARow& a_row,
                                             const BRow& b_row, const X& xtra = X()) {
    mainloop_dma_fp<FragPair<Frags<E, TM, TN, RB, TC>>, BM, BN, SPLIT, NS, NW, RB, RB, SPREAD>(
        acc, pa, pb, kbytes, kbytes, st, a_row, b_row, xtra);
}

// Mainloop with a ring of LDS stages per operand: three for the A panel, two for the B
// panel (FP: the fragments; PA, PB: the DMA panels, row-major or token-major; RB: the
// bytes of a k-tile row, 32 KB stages for 256-row panels).  The crossing at the end of k-tile j
// waits for k-tile j+1 (vmcnt(nA): only the A DMA of k-tile j+2 may be in flight),
// passes the barrier, and issues the DMA of B(j+2) and then A(j+3) into the stages j's
// own operands leave free (the first kPer instructions there, the rest over k-tile j+1's
// first SPREAD-1 k-steps), so an A k-tile is loaded two k-tiles before it is read and a
// B k-tile one.  B goes first so that the wait's in-order count never includes it.  For
// an operand that streams from HBM (each A row panel is read by few tiles at a time)
// the extra stage doubles the DMA's lead over memory latency at the same 128-byte rows.
// sa: three A stages, sb: two B stages.  K = 0 computes one k-tile of zeros; k-tiles past
// K are loaded as zeros.
// The extra loads (xtra.issue_into) go out at each crossing right after the barrier,
// before the batch, into the A stage just freed: the rows there that this wave's own
// first A instructions of the batch fill later, which lands after them (a wave's loads
// complete in order).  The next crossing's wait then covers them.
template <class FP, int NW, int RB, int SPREAD, int TM, int TN, class PA, class PB, class ARow, class BRow,
          class X = NoExtra>
__device__ __forceinline__ void mainloop_dma_ring_fp(f32x16_t (&acc)[TM][TN], const PA& pa, const PB& pb, int kbytes,
                                                     uint8_t* const (&sa)[3], uint8_t* const (&sb)[2],
                                                     const ARow& a_row, const BRow& b_row, const X& xtra = X()) {
    constexpr int KS = FP::kSteps, kMfma = TM * TN;
    constexpr int nA = PA::kInst, nB = PB::kInst;
    constexpr int kPerTile = nA + nB;
    constexpr int kPer = (kPerTile + SPREAD - 1) / SPREAD;
    static_assert(KS >= 2 && KS % 2 == 0, "the last k-step crosses; the fragment parity repeats every k-tile");
    static_assert(SPREAD >= 1 && SPREAD <= KS, "the DMA of a batch ends before the next crossing");
    static_assert(kPer <= kMfma, "one MFMA ahead of every DMA instruction");
    static_assert(nA + kPer < 64, "vmcnt range");
    static_assert(X::kOps <= nA, "the extra loads' rows are filled by the wave's own A instructions");
    const int nk = max((kbytes + RB - 1) / RB, 1);
    FP f;
    // batch instruction q: B first (q < nB), then A
    auto issue_q = [&](int q, uint8_t* a_st, uint8_t* b_st, const auto& oa, const auto& ob) {
        if (q < nB) pb.issue_one(q, b_st, ob);
        else pa.issue_one(q - nB, a_st, oa);
    };
    // prologue: A(0), B(0), A(1), then the first share of the batch {B(1), A(2)}
    pa.issue(sa[0], 0, kbytes);
    pb.issue(sb[0], 0, kbytes);
    pa.issue(sa[1], 1, kbytes);
    auto ob = pb.base_offset(1, kbytes);
    auto oa = pa.base_offset(2, kbytes);
    static_for<kPer>([&](auto Q) { issue_q(decltype(Q)::value, sa[2], sb[1], oa, ob); });
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(nA + kPer));   // A(0) and B(0) landed
    __syncthreads();
    f.load(0, sa[0], sb[0], 0, a_row, b_row);
    // stages of k-tile j: A in a_cur, B in b_cur; j+1's in a_nxt / b_nxt; the pending
    // batch (B(j+1), A(j+2)) goes to b_nxt / a_nn
    uint8_t* a_cur = sa[0];
    uint8_t* a_nxt = sa[1];
    uint8_t* a_nn = sa[2];
    uint8_t* b_cur = sb[0];
    uint8_t* b_nxt = sb[1];
    auto ktile = [&](auto FirstC, int j) {
        constexpr bool kFirst = decltype(FirstC)::value;
        static_for<KS - 1>([&](auto Sc) {
            constexpr int s = decltype(Sc)::value;
            static_for<kMfma>([&](auto J) {
                constexpr int jj = decltype(J)::value;
                f.template mma_one<kFirst && s == 0>(s & 1, jj, acc);
                if constexpr (s + 1 < SPREAD && jj < kPer && (s + 1) * kPer + jj < kPerTile)
                    issue_q((s + 1) * kPer + jj, a_nn, b_nxt, oa, ob);
                f.template slot<jj>((s + 1) & 1, a_cur, b_cur, s + 1, a_row, b_row);
                __builtin_amdgcn_sched_barrier(0);
            });
        });
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(nA));   // k-tile j+1 landed (A(j+2) may be in flight)
        __syncthreads();                              // ... for every wave; j's stages are free
        __builtin_amdgcn_sched_barrier(0);
        xtra.issue_into(j, nk, a_cur);
        ob = pb.base_offset(j + 2, kbytes);
        oa = pa.base_offset(j + 3, kbytes);
        static_for<kMfma>([&](auto J) {
            constexpr int jj = decltype(J)::value;
            f.mma_one((KS - 1) & 1, jj, acc);
            if constexpr (jj < kPer) issue_q(jj, a_cur, b_cur, oa, ob);
            f.template slot<jj>(KS & 1, a_nxt, b_nxt, 0, a_row, b_row);
            __builtin_amdgcn_sched_barrier(0);
        });
        uint8_t* const a_old = a_cur;
        a_cur = a_nxt;
        a_nxt = a_nn;
        a_nn = a_old;
        uint8_t* const b_old = b_cur;
        b_cur = b_nxt;
        b_nxt = b_old;
    };
    ktile(std::true_type{}, 0);
    for (int j = 1; j < nk; ++j) ktile(std::false_type{}, j);
    // drain the DMA that ran past the end before the LDS is reused or released
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
}

// Both operands of one element type E with RB-byte k-tile rows.
template <Elt E, int BM, int BN, int NW, int RB, int SPREAD, int TM, int TN, class ARow, class BRow,
          class X = NoExtra>
__device__ __forceinline__ void mainloop_dma_ring(f32x16_t (&acc)[TM][TN], const DmaPanel<BM, BM, NW, RB>& pa,
                                                  const DmaPanel<BN, BN, NW, RB>& pb, int kbytes,
                                                  uint8_t* const (&sa)[3], uint8_t* const (&sb)[2],
                                                  const ARow& a_row, const BRow& b_row, const X& xtra = X()) {
    mainloop_dma_ring_fp<FragPair<Frags<E, TM, TN, RB>>, NW, RB, SPREAD>(acc, pa, pb, kbytes, sa, sb, a_row, b_row,
                                                                        xtra);
}

// ---------------------------------------------------------------------------------
// Register-staged variant: global -> VGPR -> LDS.
//
// The same panels, stage layout (swz) and fragments as above, but every lane loads its
// 16-byte chunks into registers (buffer_load_dwordx4, range-checked like the DMA) and
// writes them to LDS with ds_write_b128.  The registers form a third stage ahead of the
// two LDS stages, so a tile's global loads are issued one full tile before they are
// written to LDS, and each load is waited for individually, right before its write,
// instead of all of them at the barrier.
template <int R, int SPLIT, int NW, int RB>
struct RegPanel {
    static constexpr int kCpr = RB / 16;
    static constexpr int kRpi = 1024 / RB;
    static constexpr int kRowsPerInst = kRpi * NW;
    static_assert(R % kRowsPerInst == 0 && SPLIT % kRowsPerInst == 0 && SPLIT <= R, "panel geometry");
    static constexpr int kInst = R / kRowsPerInst;  // loads per wave per k-tile
    static constexpr int kSplitInst = SPLIT / kRowsPerInst;
    __amdgpu_buffer_rsrc_t rsrc[2];
    uint32_t off0;        // byte offset of this lane's chunk in load 0 at k-tile 0
    uint32_t chunk_byte;
    uint32_t stride;      // bytes between load j and j+1 (same segment)
    int lds0;             // LDS offset (in a stage panel) of this lane's chunk in load 0

    __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
        const uint64_t p = reinterpret_cast<uint64_t>(base);
        const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
        const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
        const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
        void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
        return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, static_cast<int>(n), 0x00020000);
    }
    __device__ __forceinline__ void init(const uint8_t* seg_base0, int seg_rows0,
                                         const uint8_t* seg_base1, int seg_rows1, int kbytes) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rsrc[0] = rsrc_of(seg_base0, static_cast<uint32_t>(max(seg_rows0, 0)) * kbytes);
        rsrc[1] = rsrc_of(seg_base1, static_cast<uint32_t>(max(seg_rows1, 0)) * kbytes);
        // load j of this lane: row (NW*j + wave) * kRpi + lane / kCpr, chunk lane % kCpr;
        // the swizzle phase of the row does not depend on j (NW*kRpi rows apart)
        const int r = wave * kRpi + lane / kCpr;
        const int chunk = lane % kCpr;
        chunk_byte = static_cast<uint32_t>(chunk) << 4;
        off0 = static_cast<uint32_t>(r) * kbytes + chunk_byte;
        stride = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(kRowsPerInst) * static_cast<uint32_t>(kbytes));
        lds0 = swz<RB>(r, chunk);
    }
    __device__ __forceinline__ uint32_t base_offset(int kt, int kbytes) const {
        const uint32_t kb = static_cast<uint32_t>(kt) * RB;
        const bool kin = kb + chunk_byte < static_cast<uint32_t>(kbytes);
        uint32_t base = kin ? off0 + kb : kOob;
        asm volatile("" : "+v"(base));
        return base;
    }
    __device__ __forceinline__ i32x4_t load_one(int j, uint32_t base) const {
        const int jj = (j < kSplitInst) ? j : j - kSplitInst;
        return __builtin_amdgcn_raw_buffer_load_b128(rsrc[(j < kSplitInst) ? 0 : 1],
                                                     base + static_cast<uint32_t>(jj) * stride, 0, 0);
    }
    __device__ __forceinline__ void store_one(int j, uint8_t* panel, const i32x4_t& v) const {
        *reinterpret_cast<i32x4_t*>(panel + lds0 + j * kRowsPerInst * RB) = v;
    }
};

// Transform of the B chunks between their register stage and LDS (register-staged
// mainloop only).  NoFold: none.  GammaFold: the RMSNorm weight folded into a raw bf16
// weight on the fly, W'[n,k] = bf16_rne(fl32(gamma[k] W[n,k])) -- the separate fold's
// arithmetic, so the LDS holds the same bits as with a pre-folded weight.  A lane's
// chunk covers the same 8 k of every B row it stages, so per k-tile it loads those 8
// gamma values once (prepare) and scales all its B chunks with them (apply).
struct NoFold {
    __device__ __forceinline__ void prepare(int) {}
    __device__ __forceinline__ i32x4_t apply(const i32x4_t& v) const { return v; }
};

template <int RB>
struct GammaFold {
    __amdgpu_buffer_rsrc_t rsrc;     // gamma, K floats
    uint32_t chunk_off;              // bytes of this lane's first k within a k-tile
    float g[8];
    __device__ __forceinline__ GammaFold(const float* gamma, int K) {
        const uint64_t p = reinterpret_cast<uint64_t>(gamma);
        const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
        const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
        void* ub = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
        rsrc = __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, K * 4, 0x00020000);
        chunk_off = static_cast<uint32_t>((threadIdx.x & 63) % (RB / 16)) * 32u;   // 8 bf16 k = 8 floats
    }
    // gamma of k-tile kt's 8 k values of this lane (zeros past K, where the weight
    // chunk reads zeros too)
    __device__ __forceinline__ void prepare(int kt) {
        const uint32_t off = static_cast<uint32_t>(kt) * (RB / 2) * 4u + chunk_off;
        const f32x4_t a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
        const f32x4_t b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 16, 0, 0));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            g[e] = a[e];
            g[4 + e] = b[e];
        }
    }
    __device__ __forceinline__ i32x4_t apply(const i32x4_t& v) const {
        i32x4_t o;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t u = static_cast<uint32_t>(v[h]);
            const float p0 = g[2 * h] * bf16_bits_to_f32(static_cast<uint16_t>(u & 0xFFFFu));
            const float p1 = g[2 * h + 1] * bf16_bits_to_f32(static_cast<uint16_t>(u >> 16));
            o[h] = static_cast<int>(pack_bf16x2(p0, p1));
        }
        return o;
    }
};

// Two LDS stages + one register stage.  Per k-tile kt (reading stage kt%2):
//   k-steps 0 .. KS-2: the registers holding tile kt+1 are written to stage (kt+1)%2
//     (free since the barrier of tile kt-1), and each register is reloaded right after
//     its write with the same chunk of tile kt+2;
//   last k-step: wait for the own LDS writes, barrier (tile kt+1 complete in LDS, stage
//     kt%2 read by every wave), then MFMAs with the reads of tile kt+1's first fragments.
template <Elt E, int BM, int BN, int SPLIT, int NW, int RB, int TM, int TN, class ARow, class BRow,
          class BFold = NoFold>
__device__ __forceinline__ void mainloop_reg(f32x16_t (&acc)[TM][TN], const RegPanel<BM, BM, NW, RB>& pa,
                                             const RegPanel<BN, SPLIT, NW, RB>& pb, int kbytes,
                                             uint8_t* const (&st)[2], const ARow& a_row,
                                             const BRow& b_row, BFold fold = BFold()) {
    using F = Frags<E, TM, TN, RB>;
    constexpr int KS = F::kSteps;
    static_assert(KS >= 2, "writes go in the k-steps before the last");
    constexpr int kMfma = TM * TN;
    constexpr int nA = RegPanel<BM, BM, NW, RB>::kInst;
    constexpr int kPerTile = nA + RegPanel<BN, SPLIT, NW, RB>::kInst;
    constexpr int kPer = (kPerTile + KS - 2) / (KS - 1);      // writes per k-step
    static_assert(2 * kPer <= kMfma + 1, "one write + load per odd MFMA slot");
    const int nk = (kbytes + RB - 1) / RB;
    const int ng = (nk + 1) / 2;
    i32x4_t g[kPerTile];
    auto load_q = [&](int q, uint32_t ba, uint32_t bb) {
        g[q] = q < nA ? pa.load_one(q, ba) : pb.load_one(q - nA, bb);
    };
    auto store_q = [&](int q, uint8_t* stage) {
        if (q < nA) pa.store_one(q, stage, g[q]);
        else pb.store_one(q - nA, stage + BM * RB, fold.apply(g[q]));
    };
    F f[2];
    {
        uint32_t ba = pa.base_offset(0, kbytes), bb = pb.base_offset(0, kbytes);
        fold.prepare(0);
        static_for<kPerTile>([&](auto Q) { load_q(decltype(Q)::value, ba, bb); });
        static_for<kPerTile>([&](auto Q) { store_q(decltype(Q)::value, st[0]); });
        ba = pa.base_offset(1, kbytes); bb = pb.base_offset(1, kbytes);
        static_for<kPerTile>([&](auto Q) { load_q(decltype(Q)::value, ba, bb); });
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    f[0].load(st[0], st[0] + BM * RB, 0, a_row, b_row);

    for (int gi = 0; gi < ng; ++gi) {
        static_for<2>([&](auto I) {
            constexpr int i = decltype(I)::value;
            constexpr int par = (i * KS) & 1;
            uint8_t* cur = st[i];
            uint8_t* nxt = st[i ^ 1];
            const int kt = gi * 2 + i;
            const uint32_t ba = pa.base_offset(kt + 2, kbytes);
            const uint32_t bb = pb.base_offset(kt + 2, kbytes);
            fold.prepare(kt + 1);                      // the registers hold tile kt+1
#pragma unroll
            for (int s = 0; s < KS - 1; ++s) {
                // MFMA j; fragment read j of k-step s+1; on odd slots, register chunk q of
                // tile kt+1 to LDS, then its reload with tile kt+2
                static_for<kMfma>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    f[(par + s) & 1].mma_one(j, acc);
                    if (j < F::kReads) f[(par + s + 1) & 1].load_one(j, cur, cur + BM * RB, s + 1, a_row, b_row);
                    if (j % 2 == 1) {
                        const int q = s * kPer + j / 2;
                        if (j / 2 < kPer && q < kPerTile) {
                            store_q(q, nxt);
                            load_q(q, ba, bb);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            static_for<kMfma>([&](auto J) {
                constexpr int j = decltype(J)::value;
                f[(par + KS - 1) & 1].mma_one(j, acc);
                if (j < F::kReads) f[(par + KS) & 1].load_one(j, nxt, nxt + BM * RB, 0, a_row, b_row);
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    }
    __syncthreads();
}

// Per-wave epilogue slab region: NW slabs of SLAB_BYTES packed into the stage buffers
// (as many per stage as fit).
template <int NS, int NW, int STAGE_BYTES, int SLAB_BYTES>
__device__ __forceinline__ uint8_t* slab_region(uint8_t* const (&st)[NS], int wave) {
    constexpr int kPer = STAGE_BYTES / SLAB_BYTES;
    static_assert(kPer >= 1 && (NW + kPer - 1) / kPer <= NS, "epilogue slabs fit the stages");
    uint8_t* p = st[0];
    static_for<NS>([&](auto I) {
        if (wave / kPer == decltype(I)::value) p = st[decltype(I)::value];
    });
    return p + (wave % kPer) * SLAB_BYTES;
}

}  // namespace coda
