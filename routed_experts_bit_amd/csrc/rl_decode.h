// Decode of the Q2B and T1 expert blocks (host + device code, so the same routine is
// exercised by a CPU unit test and runs inside the gfx950 kernels).
//
// The matrix kernels never materialise decoded weights in memory (Red Lite dev75, "Prompt
// ingestion": dequantising whole experts per chunk would write gigabytes per layer).  Each
// lane decodes a strip of consecutive values of one weight row straight into MFMA operands,
// 8 values per operand.  An operand holds the exact small integer s*c (|s*c| <= 45 for Q2B,
// <= 7 for T1) as bf16 or fp16, both exact; the fp16 block scale d is applied to the fp32
// accumulator once per 256-value block.  Strips start at multiples of 8, so an operand never
// straddles a sub-scale boundary (16 values for Q2B, 32 for T1).
//
// Two small tables (built once per work-group in LDS) carry the bit work:
//   tern[b]     T1 byte b (0..242) -> its five base-3 digits, least significant first, as
//               2-bit fields (10 bits); bytes 243..255 map to five 1-digits (value 0)
//   val[s][q]   scale s, 8-bit quad q of four 2-bit codes -> the four operands s*c as 16-bit
//               floats (64 bits).  T1: c = digit - 1 (s < 8); Q2B: c = 2q - 3 (s < 16)
// A T1 strip first turns its (up to 14) digit bytes into one 2-bit digit stream through
// `tern`, shifted so that the strip's first value is digit 0; the stream (and a Q2B strip's
// code bytes directly) is then read 8 bits = 4 values at a time through `val`.
//
// A strip is handled in two phases so that kernels can issue the loads of the next block
// long before decoding it: StripRaw::load issues aligned dword loads only (block header and
// the strip's byte window), Strip::prepare turns them into code words, Strip::frag returns
// operands.  Loads never touch a dword that holds no byte of the matrix: reads go through a
// source whose device form is a buffer resource over the matrix (out-of-range dwords read 0).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

namespace rl {

constexpr int QT_Q2B = 1;
constexpr int QT_T1 = 2;

template <int QT>
struct Fmt;
template <>
struct Fmt<QT_Q2B> {
    static constexpr int BYTES = 74;
    static constexpr int NSCALE = 16;
    static constexpr int HDR_DW = 4;  // bytes 0..9 of a block at any alignment
};
template <>
struct Fmt<QT_T1> {
    static constexpr int BYTES = 57;
    static constexpr int NSCALE = 8;
    static constexpr int HDR_DW = 2;  // bytes 0..4 of a block at any alignment
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ scalar helpers
__host__ __device__ inline float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// 16-bit float pattern of a small integer (|v| <= 45): exact in both bf16 and fp16.
template <bool F16>
__host__ __device__ inline uint32_t int_to_op16(int v) {
    float f = (float)v;
    if constexpr (F16) {
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
    } else {
        return __builtin_bit_cast(uint32_t, f) >> 16;  // low 16 bits are zero for these values
    }
}

__host__ __device__ inline uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t bytes) {
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> (8 * bytes));
}

// Bytes of `tbl` picked by the four selector bytes of `sel` (each 0..3).
__host__ __device__ inline uint32_t byte_select(uint32_t tbl, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __builtin_amdgcn_perm(0u, tbl, sel);
#else
    uint32_t r = 0;
    for (int b = 0; b < 4; ++b) r |= ((tbl >> (8 * ((sel >> (8 * b)) & 3u))) & 255u) << (8 * b);
    return r;
#endif
}

// ------------------------------------------------------------------ tables
__host__ __device__ inline uint32_t tern_entry(uint32_t b) {
    if (b > 242) return 0x155u;  // five 1-digits
    uint32_t r = 0;
    for (int i = 0; i < 5; ++i) {
        uint32_t q = b / 3u;
        r |= (b - 3u * q) << (2 * i);
        b = q;
    }
    return r;
}

// Entry `idx` = s*256 + q of the value table.
template <int QT, bool F16>
__host__ __device__ inline uint64_t val_entry(int idx) {
    const int s = idx >> 8, q = idx & 255;
    uint64_t r = 0;
    for (int i = 0; i < 4; ++i) {
        int c = (q >> (2 * i)) & 3;
        int v = QT == QT_Q2B ? s * (2 * c - 3) : s * (c - 1);
        r |= (uint64_t)int_to_op16<F16>(v) << (16 * i);
    }
    return r;
}

template <int QT>
__host__ __device__ constexpr int val_entries() {
    return Fmt<QT>::NSCALE * 256;
}

// ------------------------------------------------------------------ memory sources
// Plain pointer (host tests; device code with a padded buffer).
struct PtrSrc {
    const uint8_t* p;
    __host__ __device__ inline uint32_t dw(uint32_t off) const {
        uint32_t v;
        memcpy(&v, p + off, 4);
        return v;
    }
    __host__ __device__ inline void dw4(uint32_t off, uint32_t o[4]) const {
        for (int i = 0; i < 4; ++i) o[i] = dw(off + 4 * i);
    }
    __host__ __device__ inline void dw2(uint32_t off, uint32_t o[2]) const {
        o[0] = dw(off);
        o[1] = dw(off + 4);
    }
};

// Buffer resource over one matrix of the arena (offsets are bytes from the matrix start; the
// base is 4-byte aligned and the range is rounded up to whole dwords).
struct BufSrc {
    __amdgpu_buffer_rsrc_t r;
    __device__ inline BufSrc(const void* base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)((bytes + 3u) & ~3u), 0x00020000)) {}
    __device__ inline uint32_t dw(uint32_t off) const { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0); }
    __device__ inline void dw4(uint32_t off, uint32_t o[4]) const {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        o[0] = v[0];
        o[1] = v[1];
        o[2] = v[2];
        o[3] = v[3];
    }
    __device__ inline void dw2(uint32_t off, uint32_t o[2]) const {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        o[0] = v[0];
        o[1] = v[1];
    }
};

// ------------------------------------------------------------------ strips
// STRIP consecutive values (16, 32 or 64) of one row inside one block, starting at value vs
// (a multiple of 8).  Raw dwords: the aligned dwords of the block header and of the strip's
// byte window.
template <int QT, int STRIP>
struct StripRaw {
    static constexpr int HW = Fmt<QT>::HDR_DW;
    static constexpr int WB = QT == QT_Q2B ? STRIP / 4 : (STRIP + 4 + 4) / 5;  // window bytes
    static constexpr int WW = (WB + 3 + 3) / 4;                                // window dwords
    uint32_t h[HW];
    uint32_t w[WW];
    uint32_t hm, wm;  // misalignment (bytes) of header and window
    int vs;

    template <class Src>
    __host__ __device__ inline void load(const Src& src, uint32_t blk_off, int v) {
        vs = v;
        hm = blk_off & 3u;
        const uint32_t ha = blk_off - hm;
        if constexpr (HW == 4)
            src.dw4(ha, h);
        else
            src.dw2(ha, h);
        uint32_t woff;
        if constexpr (QT == QT_Q2B)
            woff = blk_off + 10u + (uint32_t)(v >> 2);
        else
            woff = blk_off + 5u + (uint32_t)(v / 5);
        wm = woff & 3u;
        const uint32_t wa = woff - wm;
        if constexpr (WW >= 4) {
            src.dw4(wa, w);
            if constexpr (WW == 5) w[4] = src.dw(wa + 16);
        } else if constexpr (WW == 3) {
            src.dw2(wa, w);
            w[2] = src.dw(wa + 8);
        } else {
            src.dw2(wa, w);
        }
    }
};

template <int QT, int STRIP>
struct Strip {
    static constexpr int NFRAG = STRIP / 8;
    static constexpr int SW = (STRIP * 2 + 31) / 32;      // dwords of 2-bit codes
    static constexpr int FPS = QT == QT_T1 ? 4 : 2;       // fragments per sub-scale
    static constexpr int NSB = (NFRAG + FPS - 1) / FPS;   // sub-scales the strip touches
    uint32_t code[SW];  // 2-bit codes of values vs..vs+STRIP-1
    uint32_t sb[NSB];   // value-table row (s * 256) of each sub-scale; 0 everywhere when d = 0
    float d;            // block scale applied to the integer dot product

    // vs must be a multiple of min(STRIP, sub-scale span): strips never straddle a sub-scale
    // boundary except at fragment-group boundaries (true for every strip the kernels use).
    __host__ __device__ inline void prepare(const StripRaw<QT, STRIP>& raw, const uint32_t* tern) {
        const int vs = raw.vs;
        const uint32_t h0 = funnel(raw.h[1], raw.h[0], raw.hm);
        if constexpr (QT == QT_Q2B) {
            const uint32_t h1 = funnel(raw.h[2], raw.h[1], raw.hm);
            const uint32_t h2 = funnel(raw.h[3], raw.h[2], raw.hm);
            d = half_bits_to_float(h0 & 0xFFFFu) * 0.5f;
            // scale bytes 2..9 as one 64-bit word: nibble j = sub-scale of values 16j..16j+15
            const uint64_t sw = ((uint64_t)h2 << 48) | ((uint64_t)h1 << 16) | (h0 >> 16);
#pragma unroll
            for (int i = 0; i < NSB; ++i) sb[i] = (uint32_t)((sw >> (4 * ((vs >> 4) + i))) & 15u) << 8;
        } else {
            const uint32_t h1 = funnel(0u, raw.h[1], raw.hm);
            d = half_bits_to_float(h0 & 0xFFFFu);
            const uint32_t sw = (h0 >> 16) | ((h1 & 255u) << 16);
#pragma unroll
            for (int i = 0; i < NSB; ++i) sb[i] = ((sw >> (3 * ((vs >> 5) + i))) & 7u) << 8;
        }
        if (d == 0.0f) {
#pragma unroll
            for (int i = 0; i < NSB; ++i) sb[i] = 0u;  // s = 0 rows of the value table are zero
        }
        constexpr int AW = StripRaw<QT, STRIP>::WW - 1;
        uint32_t a[AW];
#pragma unroll
        for (int i = 0; i < AW; ++i) a[i] = funnel(raw.w[i + 1], raw.w[i], raw.wm);
        if constexpr (QT == QT_Q2B) {
#pragma unroll
            for (int i = 0; i < SW; ++i) code[i] = a[i];
        } else {
            const int b0 = vs / 5;
            const int r = vs - 5 * b0;
            constexpr int NB = StripRaw<QT, STRIP>::WB;
            uint32_t st[SW + 1];
#pragma unroll
            for (int i = 0; i <= SW; ++i) st[i] = 0u;
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const uint32_t c = tern[(a[i >> 2] >> (8 * (i & 3))) & 255u];
                const int bit = 10 * i;
                if (bit / 32 <= SW) st[bit / 32] |= c << (bit % 32);
                if ((bit % 32) > 22 && bit / 32 + 1 <= SW) st[bit / 32 + 1] |= c >> (32 - bit % 32);
            }
#pragma unroll
            for (int i = 0; i < SW; ++i) code[i] = (uint32_t)((((uint64_t)st[i + 1] << 32) | st[i]) >> (2 * r));
        }
    }

    // fp8 operand (32 bytes) of the 32 values vs+32h .. vs+32h+31 of a 64-value T1 strip for the
    // 16x16x128 MFMA: byte p of the operand holds value vs + 32h + pi(p) with
    //   pi(p) = 16*(p/16) + 4*(p%4) + (p/4)%4      (a 4x4 transpose inside each 16-value group),
    // so that dword q is one shift-and-mask of a code word (digits q%4, q%4+4, q%4+8, q%4+12 of
    // word 2h + q/4 as byte selectors) and one byte-select from `tbl` = [e(-s), e(0), e(+s), 0]
    // (e = the fp8 encoding).  The activation operand must use the same order.
    __host__ __device__ inline void frag8(int h, uint32_t tbl, uint32_t out[8]) const {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint32_t sel = (code[2 * h + (q >> 2)] >> (2 * (q & 3))) & 0x03030303u;
            out[q] = byte_select(tbl, sel);
        }
    }

    // operand of fragment f (values vs+8f..vs+8f+7); f must be a compile-time constant in
    // kernels so that the code words stay in registers
    __host__ __device__ inline u32x4 frag(int f, const uint64_t* val) const {
        const uint32_t w = code[f >> 1] >> (16 * (f & 1));
        const uint32_t base = sb[f / FPS];
        const uint64_t lo = val[base + (w & 255u)];
        const uint64_t hi = val[base + ((w >> 8) & 255u)];
        u32x4 r;
        r[0] = (uint32_t)lo;
        r[1] = (uint32_t)(lo >> 32);
        r[2] = (uint32_t)hi;
        r[3] = (uint32_t)(hi >> 32);
        return r;
    }
};

}  // namespace rl
