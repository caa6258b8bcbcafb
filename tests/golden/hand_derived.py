"""Writes hand_derived.json: closed-form values derived by hand from the
alpha-entmax definition and the Gaussian model (no oracle code, only math).

alpha-entmax (EntmaxKV summary, section 2; authors' abstract): exact zeros,
p_j = [(alpha-1) z_j - tau]_+^(1/(alpha-1)), sum p = 1, written here in the
scaled domain x = (alpha-1) z.  Each case carries its derivation.
Run: python tests/golden/hand_derived.py
"""
import json
import math
import os

t15 = (3 - math.sqrt(7)) / 4
D = 0.5
p1_two = (1 + D * math.sqrt(2 - D * D)) / 2

CASES = {
    "citation": "EntmaxKV summary (gist.science 2605.21649) sec. 2 (alpha-entmax, exact zeros) and "
                "sec. 2.A (bounding box, Gaussian page model); values derived by hand from the definitions",
    "entmax": [
        {"alpha": 2.0, "x": [1.0, 0.5, 0.0], "tau": 0.25, "p": [0.75, 0.25, 0.0],
         "derivation": "support {1,2}: (1-t)+(0.5-t)=1 -> t=0.25; third score 0 <= 0.25 is outside"},
        {"alpha": 1.5, "x": [1.0, 0.5, 0.0], "tau": t15, "p": [(1 - t15) ** 2, (0.5 - t15) ** 2, 0.0],
         "derivation": "support {1,2}: (1-t)^2+(0.5-t)^2=1 -> 2t^2-3t+0.25=0 -> t=(3-sqrt 7)/4; third score 0 <= t"},
        {"alpha": 2.0, "x": [2.0, 0.0, 0.0], "tau": 1.0, "p": [1.0, 0.0, 0.0],
         "derivation": "support {1}: 2-t=1 -> t=1; the zeros are <= 1"},
        {"alpha": 2.0, "x": [3.0, 3.0, 3.0, 3.0], "tau": 2.75, "p": [0.25] * 4,
         "derivation": "four equal scores: 4(3-t)=1 -> t=2.75"},
        {"alpha": 1.5, "x": [3.0, 3.0, 3.0, 3.0], "tau": 2.5, "p": [0.25] * 4,
         "derivation": "four equal scores: 4(3-t)^2=1 -> t=2.5"},
        {"alpha": 1.5, "x": [0.5, 0.0], "tau": 0.5 - math.sqrt(p1_two), "p": [p1_two, 1 - p1_two],
         "derivation": "gap D=0.5: sqrt(p1)-sqrt(p2)=D, p1+p2=1 -> p1=(1+D sqrt(2-D^2))/2; t=0.5-sqrt(p1)"},
    ],
    "bbox": [
        {"q": [1.0, -2.0], "keys": [[0.5, 1.0], [-1.0, 0.25]], "scale": 1.0,
         "kmin": [-1.0, 0.25], "kmax": [0.5, 1.0], "bound": 0.0, "token_scores": [-1.5, -1.5],
         "derivation": "box [-1,0.5]x[0.25,1]; q1>0 takes kmax_1=0.5, q2<0 takes kmin_2=0.25: 0.5-0.5=0"},
    ],
    "gauss_page": [
        {"alpha": 1.5, "scale": 0.5, "q": [2.0, 1.0], "keys": [[1.0, 3.0], [-1.0, 3.0]],
         "mean_y": 0.75, "sd_y": 0.5, "e_hat": 0.75 + 0.5 * math.sqrt(2 * math.log(2)),
         "token_scores": [1.25, 0.25],
         "derivation": "page mean (0,3), population variance (1,0); (alpha-1) scale = 0.25; "
                       "mean_Y = 0.25 (2*0 + 1*3) = 0.75; var_Y = 0.25^2 (2^2*1 + 1^2*0) = 0.25, sd_Y = 0.5; "
                       "e_hat = mean_Y + sd_Y sqrt(2 ln 2); the two token scores 0.25(2+3) = 1.25 and "
                       "0.25(-2+3) = 0.25 have mean 0.75 and population variance 0.25"},
    ],
    "gauss": [
        {"alpha": 2.0, "mu": 0.0, "sd": 1.0, "t": 0.0, "E": 1.0 / math.sqrt(2 * math.pi),
         "derivation": "E[Y_+] for a standard normal is phi(0)"},
        {"alpha": 1.5, "mu": 0.0, "sd": 1.0, "t": 0.0, "E": 0.5,
         "derivation": "E[Y_+^2] for a standard normal is E[Y^2]/2 by symmetry"},
        {"alpha": 2.0, "mu": 1.0, "sd": 0.0, "t": 0.25, "E": 0.75,
         "derivation": "zero-variance page: (1-0.25)_+"},
    ],
}

if __name__ == "__main__":
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hand_derived.json")
    with open(path, "w") as f:
        json.dump(CASES, f, indent=1)
