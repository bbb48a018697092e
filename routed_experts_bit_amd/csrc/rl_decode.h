// Decode of the Q2B and T1 expert blocks (host + device code, no intrinsics, so the same
// routine is exercised by a CPU unit test and runs inside the gfx950 kernels).
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
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rl {

constexpr int QT_Q2B = 1;
constexpr int QT_T1 = 2;

template <int QT>
struct Fmt;
template <>
struct Fmt<QT_Q2B> {
    static constexpr int BYTES = 74;
    static constexpr int NSCALE = 16;
};
template <>
struct Fmt<QT_T1> {
    static constexpr int BYTES = 57;
    static constexpr int NSCALE = 8;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// ------------------------------------------------------------------ byte windows
// Bytes p[0..nb) as little-endian dwords out[0..(nb+3)/4), loading only the aligned dwords
// that contain at least one requested byte (so a window never reads past the dword that
// holds the last byte of the arena).
template <int MAXW>
__host__ __device__ inline void load_window(const uint8_t* p, int nb, uint32_t out[MAXW]) {
    const uintptr_t a = (uintptr_t)p;
    const uint32_t* base = (const uint32_t*)(a & ~(uintptr_t)3);
    const int m = (int)(a & 3);
    const int ndw = (m + nb + 3) >> 2;
    uint32_t dw[MAXW + 1];
#pragma unroll
    for (int i = 0; i <= MAXW; ++i) dw[i] = i < ndw ? base[i] : 0u;
#pragma unroll
    for (int i = 0; i < MAXW; ++i) {
        uint64_t pair = ((uint64_t)dw[i + 1] << 32) | dw[i];
        out[i] = (uint32_t)(pair >> (8 * m));
    }
}

__host__ __device__ inline uint32_t byte_of(const uint32_t* w, int i) { return (w[i >> 2] >> (8 * (i & 3))) & 255u; }

// ------------------------------------------------------------------ strip decoder
// A strip: STRIP consecutive values (STRIP in {16, 32, 64}) of one row inside one block,
// starting at value vs (a multiple of 8).  After `load` and `prepare`, frag(f) returns the
// operand of values vs+8f .. vs+8f+7 (value vs+8f+i in 16-bit element i).
template <int QT, bool F16, int STRIP>
struct Strip {
    static constexpr int NFRAG = STRIP / 8;
    static constexpr int TB = (STRIP + 4 + 4) / 5 + 1;  // T1 digit bytes loaded (>= needed)
    static constexpr int TW = (TB + 3) / 4 + 1;         // their dwords
    static constexpr int SW = (STRIP * 2 + 31) / 32;    // dwords of the shifted digit stream
    const uint8_t* blk;
    int vs;
    uint32_t hdr[3];    // block bytes 0..9 (Q2B: d + 16 scales; T1: d + scale word)
    uint32_t raw[TW];   // T1 digit bytes / Q2B code bytes of the strip
    uint32_t code[SW];  // 2-bit codes of values vs.. (T1 after the stream shift)

    __host__ __device__ inline void load(const uint8_t* b, int v) {
        blk = b;
        vs = v;
        if constexpr (QT == QT_Q2B) {
            load_window<3>(b, 10, hdr);
            load_window<TW>(b + 10 + (v >> 2), STRIP / 4, raw);
        } else {
            load_window<3>(b, 5, hdr);
            const int b0 = v / 5;
            const int last = (v + STRIP - 1) / 5;
            load_window<TW>(b + 5 + b0, last - b0 + 1, raw);
        }
    }

    __host__ __device__ inline float scale() const {
        float d = half_bits_to_float(hdr[0] & 0xFFFFu);
        return QT == QT_Q2B ? d * 0.5f : d;
    }

    __host__ __device__ inline int subscale(int f) const {
        const int v = vs + 8 * f;
        if constexpr (QT == QT_Q2B) {
            const int j = v >> 4;
            return (int)((byte_of(hdr, 2 + (j >> 1)) >> (4 * (j & 1))) & 15u);
        } else {
            const uint32_t sc = (hdr[0] >> 16) | ((hdr[1] & 255u) << 16);
            return (int)((sc >> (3 * (v >> 5))) & 7u);
        }
    }

    // T1: digit stream through the tern table; Q2B: the code bytes are the stream.
    __host__ __device__ inline void prepare(const uint32_t* tern) {
        if constexpr (QT == QT_Q2B) {
#pragma unroll
            for (int i = 0; i < SW; ++i) code[i] = raw[i];
        } else {
            const int b0 = vs / 5;
            const int r = vs - 5 * b0;
            const int nb = (vs + STRIP - 1) / 5 - b0 + 1;
            uint32_t st[SW + 1];
#pragma unroll
            for (int i = 0; i <= SW; ++i) st[i] = 0u;
#pragma unroll
            for (int i = 0; i < TB; ++i) {
                if (i < nb) {
                    const uint32_t c = tern[byte_of(raw, i)];
                    const int bit = 10 * i;
                    if (bit / 32 <= SW) st[bit / 32] |= c << (bit % 32);
                    if ((bit % 32) > 22 && bit / 32 + 1 <= SW) st[bit / 32 + 1] |= c >> (32 - bit % 32);
                }
            }
#pragma unroll
            for (int i = 0; i < SW; ++i) {
                uint64_t pair = ((uint64_t)st[i + 1] << 32) | st[i];
                code[i] = (uint32_t)(pair >> (2 * r));
            }
        }
    }

    __host__ __device__ inline u32x4 frag(int f, const uint64_t* val) const {
        const uint32_t w = code[f >> 1] >> (16 * (f & 1));
        const int sbase = subscale(f) << 8;
        const uint64_t lo = val[sbase + (int)(w & 255u)];
        const uint64_t hi = val[sbase + (int)((w >> 8) & 255u)];
        u32x4 r;
        r[0] = (uint32_t)lo;
        r[1] = (uint32_t)(lo >> 32);
        r[2] = (uint32_t)hi;
        r[3] = (uint32_t)(hi >> 32);
        return r;
    }
};

}  // namespace rl
