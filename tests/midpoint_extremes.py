"""Set extremes (min, max), fp16 numbers, whose quotient
(max - min) / (2^b - 1) lies exactly halfway between two fp16 numbers, for
b = 4 and b = 8, each one on which the fp32 quotient's last fma rounded
straight to fp16 gives the other neighbour (for b = 2 the search found no
such set).  Found by a search over fp16 pairs; the oracle pins re-derive the midpoint property in
exact rational arithmetic, and the GPU tests build keys and values on them.
"""

MIDPOINT_EXTREMES = {
    4: [(-0.0009765625, 46.625), (-0.0322265625, 46.59375), (-0.000885009765625, 1.1357421875),
        (-0.01220703125, 27.578125)],
    8: [(-0.4736328125, 835.0), (-0.00168609619140625, 6.04296875), (-0.00559234619140625, 6.0390625),
        (-0.02587890625, 471.5), (-0.27587890625, 471.25)],
}
