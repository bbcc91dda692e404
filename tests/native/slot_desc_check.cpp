// Host check of the ragged decode's per-slot load descriptors (slot_descs_128 in
// stq_internal.h): for seeded random class counts of a 128-row head, every
// non-straddling slot's descriptor gives each lane the same two 8-byte chunk
// offsets as the per-class row layout (class k rows at b_k + (p - s_k) RB_k;
// pivot 16c and 16c + 8, 8-bit 8c, 6-bit its nibble word and its 2-bit field
// word at D / 2, 4-bit and 2-bit the word holding its codes), inside the
// head's segment, and the straddle flag marks exactly the slots whose four rows
// span two classes.
#include <cstdio>
#include <cstdlib>
#include <random>
#include "stq_internal.h"
using namespace stq;
static int rowb(int k) { return class_row_bytes_d(k, 128); }
int main() {
    std::mt19937 rng(7);
    long checked = 0, straddle = 0;
    for (int it = 0; it < 20000; ++it) {
        int n[5] = {0, 0, 0, 0, 0};
        int left = 128;
        for (int k = 0; k < 4; ++k) { int x = (int)(rng() % (left + 1)); if (rng() % 3 == 0) x = 0; n[k] = x; left -= x; }
        n[4] = left;
        if (it % 7 == 0) { for (int k=0;k<5;++k) n[k]=0; n[rng()%5]=128; }
        int32_t lay[8] = {n[0], n[1], n[2], n[3], n[4], 0, 0, 0};
        int32_t d[64];
        slot_descs_128(lay, d);
        int s[5], b[5]; s[0]=0; b[0]=0;
        for (int k=1;k<5;++k){ s[k]=s[k-1]+n[k-1]; b[k]=b[k-1]+n[k-1]*rowb(k-1); }
        int seg = b[4] + n[4]*rowb(4);
        auto cls=[&](int p){return (p>=s[1])+(p>=s[2])+(p>=s[3])+(p>=s[4]);};
        for (int w=0; w<4; ++w) for (int m=0; m<8; ++m) {
            const int P = d[2*(8*w+m)+1], base = d[2*(8*w+m)];
            const bool st = cls(16*m+4*w) != cls(16*m+4*w+3);
            if (st != (P < 0)) { printf("straddle flag mismatch\n"); return 1; }
            if (P < 0) { ++straddle; continue; }
            for (int gl=0; gl<4; ++gl) for (int c=0; c<16; ++c) {
                const int g = 4*w+gl, p = g+16*m, k = cls(p);
                // reference: the per-class formulas of the kernel
                const unsigned row = (unsigned)(b[k] + (p - s[k]) * rowb(k));
                const unsigned uc = c; unsigned A, B;
                if (k==0){A=row+16u*uc;B=A+8u;} else if(k==1){A=row+8u*uc;B=A;}
                else if(k==2){A=row+((4u*uc)&~7u);B=row+64u+((2u*uc)&~7u);}
                else if(k==3){A=row+((4u*uc)&~7u);B=A;} else {A=row+((2u*uc)&~7u);B=A;}
                // descriptor path
                const unsigned rb=(unsigned)P&0x1FFu, shA=((unsigned)P>>16)&15u, shB=((unsigned)P>>20)&15u, ob=((unsigned)P>>24)&0x7Fu;
                const unsigned kk=((unsigned)P>>9)&7u;
                const unsigned r2=(unsigned)base+(unsigned)g*rb, c2=2u*uc;
                const unsigned A2=r2+((c2>>shA)<<3), B2=r2+ob+((c2>>shB)<<3);
                if (A!=A2||B!=B2||kk!=(unsigned)k){printf("mismatch n=%d %d %d %d %d w%d m%d g%d c%d k%d: %u %u vs %u %u\n",n[0],n[1],n[2],n[3],n[4],w,m,g,c,k,A,B,A2,B2);return 1;}
                if (A2+8>(unsigned)seg||B2+8>(unsigned)seg){printf("out of segment\n");return 1;}
                ++checked;
            }
        }
    }
    printf("ok: %ld lane-slot checks, %ld straddling slots\n", checked, straddle);
    return 0;
}
