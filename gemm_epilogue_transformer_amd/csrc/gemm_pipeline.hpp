// Direct-to-LDS MFMA mainloop (gfx950) shared by both GEMM kernels of the chain.
//
// Block tile BM x BN, 4 waves in a 2 x 2 grid, each wave owning (BM/2) x (BN/2) made of
// 32x32 MFMA blocks.  A k-tile is 64 bytes of every row (32 bf16 or 64 e4m3 values).
//
// Global -> LDS: `buffer_load_dwordx4 ... lds` moves 16 bytes per lane straight into
// LDS (no VGPR staging).  One instruction fills 1 KB = 16 consecutive panel rows of 64
// bytes: lane i lands at LDS byte 16*i of that 1 KB, i.e. row i/4, slot i%4.
//
// LDS layout: 16-byte chunk c of row r sits in slot c ^ ((r >> 2) & 3).  The LDS has 64
// banks (256 bytes) and serves a ds_read_b128 16 lanes at a time; the 16 lanes of a
// fragment read touch 16 consecutive rows at one chunk, and the swizzle spreads them over
// all 16 distinct 16-byte bank groups.  On the DMA side lane i therefore FETCHES chunk
// (i%4) ^ ((i/16) & 3) of its row.
//
// Rows past the matrix and chunks past K read as zero through the buffer descriptor's
// range check (each descriptor spans exactly the valid rows of one row segment; K-tail
// chunks get an offset beyond every range).
//
// Pipeline: 4 LDS stages in 4 distinct __shared__ arrays (so the compiler can tell the
// DMA into one stage from the fragment reads of another), DMA running 3 k-tiles ahead.
// Per k-tile: wait until this tile's DMA has landed (the 2 younger tiles may still be in
// flight), barrier, issue the DMA of tile kt+3 into the stage freed by tile kt-1, MFMAs.
#pragma once

#include <type_traits>

#include "gemm_core.hpp"

namespace coda {

constexpr int kTileBytes = 64;          // bytes of one row per k-tile
constexpr int kStages = 4;
constexpr uint32_t kOob = 0x80000000u;  // offset that no descriptor range reaches

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kTileBytes + ((chunk ^ ((row >> 2) & 3)) << 4);
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
// for a single segment).  Instruction j of wave w covers panel rows [(4j + w) * 16, +16),
// so with SPLIT % 64 == 0 every instruction stays inside one segment and the segment of
// instruction j is j < SPLIT/64.
template <int R, int SPLIT>
struct DmaPanel {
    static_assert(R % 64 == 0 && SPLIT % 64 == 0 && SPLIT <= R, "panel geometry");
    static constexpr int kInst = R / 64;           // DMA instructions per wave per k-tile
    u32x4_t rsrc[2];
    uint32_t off0;            // byte offset of this lane's chunk in instruction 0 at k-tile 0
    uint32_t chunk_byte;      // 16 * the chunk this lane fetches
    uint32_t stride;          // bytes between instruction j and j+1 (64 rows), wave-uniform

    // seg_base[s]: address of the segment's first row; seg_rows[s]: rows of the segment that
    // exist in the matrix (the descriptor range); kbytes: bytes of one matrix row.
    __device__ __forceinline__ void init(const uint8_t* seg_base0, int seg_rows0,
                                         const uint8_t* seg_base1, int seg_rows1, int kbytes) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rsrc[0] = make_rsrc(seg_base0, static_cast<uint32_t>(max(seg_rows0, 0)) * kbytes);
        rsrc[1] = make_rsrc(seg_base1, static_cast<uint32_t>(max(seg_rows1, 0)) * kbytes);
        chunk_byte = static_cast<uint32_t>((lane & 3) ^ ((lane >> 4) & 3)) << 4;
        off0 = static_cast<uint32_t>(wave * 16 + (lane >> 2)) * kbytes + chunk_byte;
        stride = __builtin_amdgcn_readfirstlane(64u * static_cast<uint32_t>(kbytes));
    }

    // Issue the DMA of k-tile kt into `stage` (R rows x 64 bytes).  Row of instruction j,
    // lane l: (4j + wave) * 16 + l/4; segment-1 rows are rebased by SPLIT.
    __device__ __forceinline__ void issue(uint8_t* stage, int kt, int kbytes) const {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const uint32_t kb = static_cast<uint32_t>(kt) * kTileBytes;
        // a chunk past K starts from kOob: kOob + jj*stride stays beyond every range
        // (each descriptor spans < 2^31 bytes), so the whole lane reads zeros
        const bool kin = kb + chunk_byte < static_cast<uint32_t>(kbytes);
        uint32_t base = kin ? off0 + kb : kOob;
        // keep the per-instruction offsets derived here (not hoisted as kInst live registers)
        asm volatile("" : "+v"(base));
#pragma unroll
        for (int j = 0; j < kInst; ++j) {
            const int row0 = (4 * j + wave) * 16;
            const int jj = (j < SPLIT / 64) ? j : j - SPLIT / 64;
            const uint32_t voff = base + static_cast<uint32_t>(jj) * stride;
            dma16(rsrc[(j < SPLIT / 64) ? 0 : 1], voff, lds_addr(stage + row0 * kTileBytes));
        }
    }
};

// Fragments of one MFMA k-step for a wave's TM x TN 32x32 blocks.  bf16: a k-step is
// k16 (2 per k-tile), one 16-byte ds_read per fragment.  e4m3: a k-step is k64 (1 per
// k-tile), two 16-byte ds_reads per fragment.
template <Elt E, int TM, int TN>
struct Frags;

template <int TM, int TN>
struct Frags<Elt::BF16, TM, TN> {
    static constexpr int kSteps = 2;
    static constexpr int kReads = TM + TN;         // ds_read_b128 per k-step
    bf16x8_t a[TM], b[TN];
    template <class ARow, class BRow>
    __device__ __forceinline__ void load(const uint8_t* sA, const uint8_t* sB, int s,
                                         const ARow& a_row, const BRow& b_row) {
        const int lane = threadIdx.x & 63;
        const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
            a[tm] = *reinterpret_cast<const bf16x8_t*>(sA + swz(a_row(tm) + lr, 2 * s + lh));
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
            b[tn] = *reinterpret_cast<const bf16x8_t*>(sB + swz(b_row(tn) + lr, 2 * s + lh));
    }
    __device__ __forceinline__ void mma(f32x16_t (&acc)[TM][TN]) const {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[tm], b[tn], acc[tm][tn], 0, 0, 0);
    }
};

template <int TM, int TN>
struct Frags<Elt::E4M3, TM, TN> {
    static constexpr int kSteps = 1;
    static constexpr int kReads = 2 * (TM + TN);
    i32x8_t a[TM], b[TN];
    template <class ARow, class BRow>
    __device__ __forceinline__ void load(const uint8_t* sA, const uint8_t* sB, int,
                                         const ARow& a_row, const BRow& b_row) {
        const int lane = threadIdx.x & 63;
        const int lr = lane & 31, lh = lane >> 5;
        // lane holds 32 bytes of its row = chunks 2*lh, 2*lh+1
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            const int row = a_row(tm) + lr;
            const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(sA + swz(row, 2 * lh));
            const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(sA + swz(row, 2 * lh + 1));
            a[tm] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const int row = b_row(tn) + lr;
            const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(sB + swz(row, 2 * lh));
            const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(sB + swz(row, 2 * lh + 1));
            b[tn] = i32x8_t{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    }
    __device__ __forceinline__ void mma(f32x16_t (&acc)[TM][TN]) const {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
                // formats 0/0 = e4m3 x e4m3; block scales 127 = 2^0 (unscaled)
                acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    a[tm], b[tn], acc[tm][tn], 0, 0, 0, 127, 0, 127);
    }
};

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14]); expcnt / lgkmcnt are left at their maxima.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Instruction classes for the scheduler hints (llvm.amdgcn.sched.group.barrier masks).
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

// Interleave `n_mfma` MFMAs with `n_ds` LDS reads and `n_vm` global->LDS loads: one MFMA,
// then one of each memory op, while they last; the remaining MFMAs follow.
template <int N_MFMA, int N_DS, int N_VM>
__device__ __forceinline__ void sched_interleave() {
    constexpr int kMem = N_DS > N_VM ? N_DS : N_VM;
#pragma unroll
    for (int i = 0; i < kMem; ++i) {
        if (i < N_MFMA) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if (i < N_VM) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
        if (i < N_DS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    if (N_MFMA > kMem) __builtin_amdgcn_sched_group_barrier(kSchedMfma, N_MFMA - kMem, 0);
}

// The whole mainloop: acc += A_panel . B_panel^T over the k-tiles of one row.
// st0..st3 are the four stage buffers, each (BM + BN) * 64 bytes.
//
// Software pipeline (per wave).  Fragments are double-buffered by MFMA k-step: the
// fragments of step j+1 are read from LDS while the MFMAs of step j run.  The last
// k-step of tile kt is where the next tile's first fragments are needed, so that is
// where the wave waits for tile kt+1's DMA, passes the barrier (after which every wave
// has also finished reading tile kt-1, whose stage receives the DMA of tile kt+3), issues
// that DMA and reads tile kt+1's first fragments, all interleaved with the MFMAs.
template <Elt E, int BM, int BN, int SPLIT, int TM, int TN, class ARow, class BRow>
__device__ __forceinline__ void mainloop_dma(f32x16_t (&acc)[TM][TN], const DmaPanel<BM, BM>& pa,
                                             const DmaPanel<BN, SPLIT>& pb, int kbytes,
                                             uint8_t* st0, uint8_t* st1, uint8_t* st2,
                                             uint8_t* st3, const ARow& a_row, const BRow& b_row) {
    using F = Frags<E, TM, TN>;
    constexpr int KS = F::kSteps;
    constexpr int kMfma = TM * TN;
    // DMA instructions per wave per k-tile; when tile kt+1 must have landed, only tile
    // kt+2 is younger, so kPerTile DMA instructions may stay in flight
    constexpr int kPerTile = DmaPanel<BM, BM>::kInst + DmaPanel<BN, SPLIT>::kInst;
    static_assert(2 * kPerTile < 64, "vmcnt range");
    const int nk = (kbytes + kTileBytes - 1) / kTileBytes;
    // k-tiles run in groups of 4 (one per stage); the count is padded to a multiple of 4
    // with k-tiles past K, which the DMA fills with zeros.  The DMA always runs 3 tiles
    // ahead, past the padded end too (zeros into stages that are not read again), so the
    // wait counts are exact on every tile.
    const int nq = (nk + 3) >> 2;
    auto issue = [&](uint8_t* st, int kt) {
        pa.issue(st, kt, kbytes);
        pb.issue(st + BM * kTileBytes, kt, kbytes);
    };
    F f[2];
    issue(st0, 0);
    issue(st1, 1);
    issue(st2, 2);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kPerTile));   // tile 0 landed
    __syncthreads();
    f[0].load(st0, st0 + BM * kTileBytes, 0, a_row, b_row);

    // one k-tile in stage `cur`; `nxt` holds tile kt+1, `dst` receives the DMA of kt+3.
    // G = global k-step index parity base (k-steps of this tile use f[(G + s) & 1]).
    auto tile = [&](auto G, uint8_t* cur, uint8_t* nxt, uint8_t* dst, int kt) {
        constexpr int g = decltype(G)::value;
#pragma unroll
        for (int s = 0; s < KS - 1; ++s) {
            f[(g + s + 1) & 1].load(cur, cur + BM * kTileBytes, s + 1, a_row, b_row);
            f[(g + s) & 1].mma(acc);
            sched_interleave<kMfma, F::kReads, 0>();
            __builtin_amdgcn_sched_barrier(0);
        }
        // last k-step of the tile: cross into tile kt+1
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(kPerTile));   // tile kt+1 landed (this wave)
        __syncthreads();                                    // ... for every wave
        __builtin_amdgcn_sched_barrier(0);
        issue(dst, kt + 3);
        f[(g + KS) & 1].load(nxt, nxt + BM * kTileBytes, 0, a_row, b_row);
        f[(g + KS - 1) & 1].mma(acc);
        sched_interleave<kMfma, F::kReads, 0>();
        __builtin_amdgcn_sched_barrier(0);
    };
    using G0 = std::integral_constant<int, 0>;
    using G1 = std::integral_constant<int, KS & 1>;
    using G2 = std::integral_constant<int, 0>;
    using G3 = std::integral_constant<int, KS & 1>;
    for (int q = 0; q < nq; ++q) {
        const int kt = 4 * q;
        tile(G0{}, st0, st1, st3, kt);
        tile(G1{}, st1, st2, st0, kt + 1);
        tile(G2{}, st2, st3, st1, kt + 2);
        tile(G3{}, st3, st0, st2, kt + 3);
    }
    // drain the DMA that ran past the end before the LDS is reused or released
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
}

}  // namespace coda
