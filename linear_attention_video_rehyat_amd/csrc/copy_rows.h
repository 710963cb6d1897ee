// copy_rows.h -- one 16-byte piece of the streaming overlap copy (device code).
#pragma once
#include "common.h"
#include "kernels.h"

namespace rehyat {

// Piece idx of the kept rows: row r of (b, h) is virtual row
// prev_rows + chunk_rows - keep_rows + r of [prev | chunk]; d * elem_bytes / 16
// pieces per row (cpr).
__device__ __forceinline__ void prev_copy_chunk(const PrevCopyParams& p, const int cpr, const long long idx) {
    const int c = (int)(idx % cpr);
    const long long rr = idx / cpr;
    const int r = (int)(rr % p.keep_rows);
    const int bh = (int)(rr / p.keep_rows);
    const int j = p.prev_rows + p.chunk_rows - p.keep_rows + r;
    const char* ks;
    const char* vs;
    const long long rowb = (long long)p.d * p.elem_bytes;
    if (j < p.prev_rows) {
        ks = (const char*)p.kp + ((long long)bh * p.prev_bh_stride) * p.elem_bytes + j * rowb;
        vs = (const char*)p.vp + ((long long)bh * p.prev_bh_stride) * p.elem_bytes + j * rowb;
    } else {
        ks = (const char*)p.k + ((long long)bh * p.bh_stride) * p.elem_bytes + (j - p.prev_rows) * rowb;
        vs = (const char*)p.v + ((long long)bh * p.bh_stride) * p.elem_bytes + (j - p.prev_rows) * rowb;
    }
    const long long doff = ((long long)bh * p.prev_bh_stride) * p.elem_bytes + r * rowb + 16LL * c;
    *(u32x4*)((char*)p.kd + doff) = *(const u32x4*)(ks + 16LL * c);
    if (p.vd) *(u32x4*)((char*)p.vd + doff) = *(const u32x4*)(vs + 16LL * c);
}

}  // namespace rehyat
