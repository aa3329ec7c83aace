// Packed-tile geometry and the HBM -> LDS / LDS -> MFMA helpers of the bf16 attention kernel.
#pragma once

#include <type_traits>

#include "kernels.hpp"

namespace spark {

constexpr int kTK = 64;  // keys per tile

template <int D> struct TileGeom {
    static constexpr int CK = D / 8;                  // 16-byte chunks per K row
    static constexpr int ELEMS = 2 * kTK * D;         // bf16 elements of a packed tile
    static constexpr int CHUNKS = ELEMS / 8;          // 16-byte chunks of a packed tile
    static constexpr int K_CHUNKS = kTK * CK;         // chunks of the K part
    static constexpr int V_CPR = kTK / 8;             // chunks per V^T row (8)
};

// Chunk swizzle of an LDS row: rows of 16 chunks (256 B) use row % 16; rows of 8 chunks (128 B)
// use (row / 2) % 8, so 16 consecutive rows read at one logical chunk hit 16 distinct bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    return CPR == 16 ? (row & 15) : ((row >> 1) & 7);
}

// Row order of K inside each 32-key group: swap bits 2 and 3.
__device__ __forceinline__ int key_perm(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// Source chunks (16 bytes) of a packed tile for LDS chunk q: K rows in the order pi with the row
// swizzle (K part), V^T rows with theirs (V part).  They depend only on q, so every lane computes
// its offsets once.
template <int D>
__device__ __forceinline__ int k_src_chunk(int q) {
    using G = TileGeom<D>;
    const int m = q / G::CK, pc = q % G::CK;
    const int grow = (m & ~31) | key_perm(m & 31);
    return grow * G::CK + (pc ^ swz<G::CK>(m));
}
template <int D>
__device__ __forceinline__ int v_src_chunk(int q) {
    using G = TileGeom<D>;
    const int dr = q / G::V_CPR, pc = q % G::V_CPR;
    return G::K_CHUNKS + dr * G::V_CPR + (pc ^ swz<G::V_CPR>(dr));
}

// HBM -> LDS copy of one half (K rows, or V^T rows) of a packed tile with buffer_load ... lds: every
// lane moves NCH 16-byte chunks.  Chunk i of a lane is LDS chunk i*NT + tid, whose source chunk is
// src(i*NT + tid).  Where src(i*NT + tid) = src(tid) + i*NT (every shape but d = 128 with 64-row
// query blocks) a lane keeps one 32-bit byte offset and the chunk term goes into the scalar offset;
// otherwise one offset per chunk.  The LDS destination of a wave's 64 chunks is contiguous (lane l
// writes base + 16 l), the base is a scalar (M0).
template <int D, int NT> struct DmaPlan {
    static constexpr int NCH = TileGeom<D>::K_CHUNKS / NT;
    static constexpr bool kAffine = (NT / TileGeom<D>::CK) % 16 == 0;
    static constexpr int NOFF = kAffine ? 1 : NCH;
};

// Buffer resource of a byte range (CDNA3/CDNA4 ISA, buffer resource descriptor: base, zero stride,
// size in bytes for the range check, word 3 as for untyped 32-bit data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int D, int NT, typename RS>
__device__ __forceinline__ void issue_half(RS rs, uint32_t tile_byte,
                                           const uint32_t (&off)[DmaPlan<D, NT>::NOFF], __bf16* l, int wv) {
    using PL = DmaPlan<D, NT>;
#pragma unroll
    for (int i = 0; i < PL::NCH; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(l + (size_t)(i * NT + wv * 64) * 8), 16,
                                                 PL::kAffine ? off[0] : off[i],
                                                 tile_byte + (PL::kAffine ? (uint32_t)(i * NT * 16) : 0u), 0, 0);
}

// S^T = K_tile Q^T for two chunks of 32 keys x this wave's 32 queries.  kboff[ds]: byte offset of
// lane (i32, h)'s A operand in row i32 of the tile for k step ds (row 32 + i32 is 64*D bytes further).
// The accumulators start at `init` (zero, or -U on the fixed-offset pass).
template <int D>
__device__ __forceinline__ void scores(const __bf16* Kl, const uint32_t (&kboff)[D / 16],
                                       const bf16x8 (&qreg)[D / 16], const f32x16& init, f32x16 (&st)[2]) {
    const char* Kb = reinterpret_cast<const char*>(Kl);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        f32x16 a16 = init;
#pragma unroll
        for (int ds = 0; ds < D / 16; ++ds) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kb + c * 64 * D + kboff[ds]);
            a16 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ds], a16, 0, 0, 0);
        }
        st[c] = a16;
    }
}

template <int V> using IC = std::integral_constant<int, V>;

// Start value of the fixed-offset pass: pre-scaled query row (q * c_log2 rounded to bf16) for the
// B operand of S^T = K Q^T, lane (i32, h) holding dims ds*16 + 8h .. +8 of its row, and the row's
// squared norm over those dims.
template <typename T, int D>
__device__ __forceinline__ float load_q_scaled(const T* src, bool valid, float c_log2, bf16x8 (&qreg)[D / 16],
                                               int h) {
    float ss = 0.f;
#pragma unroll
    for (int ds = 0; ds < D / 16; ++ds) {
        u32x4 u = {0u, 0u, 0u, 0u};
        if (valid) {
            float v[8];
            In<T>::load8(src + ds * 16 + 8 * h, v);
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] *= c_log2;
            u = pack8_bf16(v);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo = bf16_bits_to_f32(u[j] & 0xffffu), hi = bf16_bits_to_f32(u[j] >> 16);
                ss = fmaf(lo, lo, ss);
                ss = fmaf(hi, hi, ss);
            }
        }
        qreg[ds] = __builtin_bit_cast(bf16x8, u);
    }
    return ss;
}

}  // namespace spark
